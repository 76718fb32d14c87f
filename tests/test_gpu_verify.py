"""GPU parity of the verification pass (kvq_verify_attention): the q_len newest
positions of each sequence attend causally to the quantized paged cache.

Each (sequence, position, head) row is compared with the oracle's
verify_reference on the same seeded inputs: |gpu - oracle| <= 2e-3 +
1e-2 |oracle|, lse within 1e-3; a position that sees no token must give
exactly out = 0 and lse = -inf.  q_len = 1 must equal kvq_decode_attention
bit for bit.
"""
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
LSE_ATOL = 1e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def workload(base: str, **kw) -> synthetic.Workload:
    d = dict(synthetic.WORKLOADS[base].__dict__)
    d.update(kw)
    return synthetic.Workload(**d)


def verify_q(w: synthetic.Workload, B: int, q_len: int, device) -> torch.Tensor:
    """bf16 queries [B][q_len][Hq][d] from the seeded query generator."""
    return synthetic.gen_q(w, device, batch=B * q_len).reshape(B, q_len, w.num_q_heads, w.head_dim)


def run_verify(bt: H.Built, q: torch.Tensor, partition_pages: int = 0):
    B, q_len, Hq, d = q.shape
    scale = 1.0 / math.sqrt(d)
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, q_len, Hq, bt.max_ctx, partition_pages),
                     dtype=torch.uint8, device=q.device)
    out = torch.full((B, q_len, Hq, d), float("nan"), device=q.device)
    lse = torch.full((B, q_len, Hq), float("nan"), device=q.device)
    kvq.verify_attention(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, scale, ws, out, lse,
                         partition_pages)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(bt: H.Built, q_len: int, out: np.ndarray, lse: np.ndarray, seqs=None):
    w = bt.w
    B = len(bt.lens)
    q_cpu = verify_q(w, B, q_len, "cpu")
    dt = H.oracle_dtype(w)
    for b in (range(B) if seqs is None else seqs):
        T = int(bt.lens[b])
        k, v = synthetic.gen_kv(w, b, 0, T, bt.q.device)   # bitwise device-independent
        ref = O.verify_reference(H.u16(q_cpu[b]), H.u16(k), H.u16(v), dt)
        for i in range(q_len):
            if T - q_len + 1 + i <= 0:
                assert not out[b, i].any() and np.all(np.isneginf(lse[b, i])), (b, i)
                continue
            ok, mabs, mrel = H.allclose_report(out[b, i], ref["out"][i], ATOL, RTOL)
            assert ok, f"seq {b} (len {T}) position {i}: max abs {mabs:.3e} max rel {mrel:.3e}"
            dl = np.abs(lse[b, i].astype(np.float64) - ref["lse"][i]).max()
            assert dl <= LSE_ATOL, f"seq {b} position {i}: lse diff {dl:.3e}"


LENS = np.array([1, 2, 3, 5, 16, 17, 33, 40, 100, 257, 700], dtype=np.int64)


@pytest.mark.parametrize("base,heads,q_len", [
    ("tiny", (8, 2), 2),       # FP8, group 4
    ("tiny", (8, 2), 4),       # FP8, group 4: 16 rows
    ("tiny", (4, 2), 8),       # FP8, group 2: 16 rows
    ("tiny", (2, 2), 16),      # FP8, group 1: 16 rows, one position per row
    ("llama70b", (16, 2), 2),  # INT8, group 8: 16 rows
    ("llama70b", (8, 2), 3),   # INT8, group 4: 12 rows
])
def test_verify_matches_oracle(base, heads, q_len):
    w = workload(base, num_q_heads=heads[0], num_kv_heads=heads[1], batch=len(LENS), context=int(LENS.max()))
    say("verify", base, heads, "q_len", q_len)
    bt = H.build(w, lens=LENS)
    q = verify_q(w, len(LENS), q_len, "cuda")
    for part in (0, 1, 3):
        say("  partition pages", part)
        out, lse = run_verify(bt, q, part)
        check(bt, q_len, out, lse)


def test_verify_shuffled_pages_ragged_batch():
    w = workload("mixed", batch=24, num_q_heads=8, num_kv_heads=2)
    lens = synthetic.seq_lens(w)[:24] // 8 + 1
    say("verify shuffled, lens", lens.min(), lens.max())
    bt = H.build(w, lens=lens, shuffle=True)
    q = verify_q(w, len(lens), 4, "cuda")
    out, lse = run_verify(bt, q, 0)
    check(bt, 4, out, lse)


def test_verify_one_position_is_decode_bit_for_bit():
    for base, heads in (("tiny", (8, 2)), ("llama70b", (16, 2))):
        w = workload(base, num_q_heads=heads[0], num_kv_heads=heads[1], batch=len(LENS), context=int(LENS.max()))
        say("q_len 1 vs decode", base)
        bt = H.build(w, lens=LENS)
        q = verify_q(w, len(LENS), 1, "cuda")
        bt.q = q[:, 0].contiguous()
        for part in (0, 2):
            out_d, lse_d = H.run_decode(bt, part)
            out_v, lse_v = run_verify(bt, q, part)
            assert np.array_equal(out_v[:, 0], out_d.cpu().numpy())
            assert np.array_equal(lse_v[:, 0], lse_d.cpu().numpy())


def test_verify_llama8b_shape_every_sequence():
    """The 8B-shaped batch (B 32, context 8192, FP8, 32 q / 8 KV heads) with 4
    positions per sequence, in the launch configuration the benchmark uses;
    every sequence checked row by row against the oracle."""
    w = synthetic.WORKLOADS["llama8b"]
    say("verify llama8b shape q_len 4")
    bt = H.build(w)
    q = verify_q(w, w.batch, 4, "cuda")
    out, lse = run_verify(bt, q, 0)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    check(bt, 4, out, lse)


def test_verify_split_then_reduce_equals_attention():
    w = workload("tiny", num_q_heads=8, num_kv_heads=2, batch=len(LENS), context=int(LENS.max()))
    say("verify split + reduce vs attention")
    bt = H.build(w, lens=LENS)
    B, q_len, Hq, d = len(LENS), 4, 8, 128
    q = verify_q(w, B, q_len, "cuda")
    for part in (0, 1):
        out_a, lse_a = run_verify(bt, q, part)
        ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, q_len, Hq, bt.max_ctx, part), dtype=torch.uint8,
                         device="cuda")
        out = torch.full((B, q_len, Hq, d), float("nan"), device="cuda")
        lse = torch.full((B, q_len, Hq), float("nan"), device="cuda")
        kvq.verify_split(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, 1.0 / math.sqrt(d), ws, out, lse,
                         part)
        kvq.verify_reduce(bt.cache, B, q_len, Hq, bt.max_ctx, ws, out, lse, part)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), out_a) and np.array_equal(lse.cpu().numpy(), lse_a)
