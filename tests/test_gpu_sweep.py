"""Seeded sweep over combinations of the FP8 / INT8 path's options, each checked
against the oracle: format (E4M3, E5M2, INT8), scale mode (per-token, static
per-head, static per-tensor), page size (16, 32), KV heads (1-3) and group
(1-16), query positions (decode, or a causal verification of 2-4
positions), FP8-domain QK, partition size, ragged lengths including empty
sequences and shuffled pools.  Other tests take these options one at a time;
this one checks them in combination.  The bar is the decode bar (2e-3
absolute + 1e-2 relative; FP8-domain lse per its own bound).
"""
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
N_CASES = 48


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def draw_case(rng):
    dtype = ["fp8", "e5m2", "int8"][rng.integers(3)]
    mode = kvq.KVQ_SCALE_PER_TOKEN_HEAD if dtype == "int8" else int(rng.choice([2, 2, 1, 0]))
    n_kv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    q_len = int(rng.choice([1, 1, 2, 4]))
    while G * q_len > 16:
        q_len //= 2
    q8 = dtype != "int8" and bool(rng.integers(2))
    B = int(rng.integers(1, 7))
    lens = rng.integers(0, 300, size=B)
    lens[rng.integers(B)] = max(int(lens.max()), 1)
    return dict(dtype=dtype, mode=mode, page_size=int(rng.choice([16, 32])), n_kv=n_kv, G=G, q_len=q_len,
                q8=q8, lens=lens, part=int(rng.choice([0, 0, 1, 3])), shuffle=bool(rng.integers(2)))


def static_scales(rng, mode, n_kv, dtype):
    """bf16 [2][n_kv] (per head) or [2][1] (per tensor); values around the
    inputs' spread over the format's largest code, so some codes saturate."""
    top = 57344.0 if dtype == "e5m2" else 448.0
    k = rng.uniform(4.0, 80.0, size=n_kv) / top
    v = rng.uniform(2.0, 6.0, size=n_kv) / top
    host = np.stack([k, v]).astype(np.float32)
    if mode == kvq.KVQ_SCALE_PER_TENSOR:
        host = host[:, :1]
    t = torch.from_numpy(host).to(torch.bfloat16)
    return t.cuda().contiguous(), (H.u16(t[0]), H.u16(t[1]))


@pytest.mark.parametrize("case", range(N_CASES))
def test_option_combinations(case):
    rng = np.random.default_rng(1000 + case)
    c = draw_case(rng)
    say(case, {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()})
    base = synthetic.WORKLOADS["tiny"]
    d = dict(base.__dict__)
    d.update(dtype=c["dtype"], batch=len(c["lens"]), num_q_heads=c["n_kv"] * c["G"], num_kv_heads=c["n_kv"],
             page_size=c["page_size"], context=int(c["lens"].max()), seed=7 + case)
    w = synthetic.Workload(**d)
    ss, static_kv = (None, None)
    if c["mode"] != kvq.KVQ_SCALE_PER_TOKEN_HEAD:
        ss, static_kv = static_scales(rng, c["mode"], c["n_kv"], c["dtype"])
    bt = H.build(w, lens=c["lens"], mode=c["mode"], static_scales=ss, shuffle=c["shuffle"])
    bt.cache.attn_flags = kvq.KVQ_ATTN_FP8_QK if c["q8"] else 0
    B, Hq, dh, QL = len(c["lens"]), w.num_q_heads, w.head_dim, c["q_len"]
    scale = dh ** -0.5
    q = synthetic.gen_q(w, "cuda", batch=B * QL).reshape(B, QL, Hq, dh).contiguous()
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, QL, Hq, bt.max_ctx, c["part"]), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, QL, Hq, dh), float("nan"), device="cuda")
    lse = torch.full((B, QL, Hq), float("nan"), device="cuda")
    if QL == 1:
        o1 = out[:, 0].contiguous()
        l1 = lse[:, 0].contiguous()
        kvq.decode_attention(bt.cache, q[:, 0].contiguous(), bt.block_table, bt.context_lens, bt.max_ctx, scale,
                             ws, o1, l1, c["part"])
        out, lse = o1[:, None], l1[:, None]
    else:
        kvq.verify_attention(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, scale, ws, out, lse,
                             c["part"])
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qc = synthetic.gen_q(w, "cpu", batch=B * QL).reshape(B, QL, Hq, dh)
    for b in range(B):
        T = int(c["lens"][b])
        k, v = synthetic.gen_kv(w, b, 0, T, "cpu")
        ref = O.verify_reference(H.u16(qc[b]), H.u16(k), H.u16(v), H.oracle_dtype(w), c["mode"], static_kv,
                                 scale, q8=c["q8"])
        for i in range(QL):
            if T - QL + 1 + i <= 0:
                assert not out[b, i].any() and np.all(np.isneginf(lse[b, i])), (b, i)
                continue
            ok, mabs, mrel = H.allclose_report(out[b, i], ref["out"][i], ATOL, RTOL)
            assert ok, f"seq {b} position {i}: max abs {mabs:.3e} max rel {mrel:.3e}"
            bar = 1e-3
            if c["q8"]:
                # FP8 matrix-core dot products: |d score| <= 2^-12 scale max_t sum |q^ k^|
                n_vis = T - QL + 1 + i
                qh = np.abs(O.fp8_query(H.u16(qc[b, i])))
                kh = np.abs(ref["k_hat"][:n_vis])
                mag = np.array([(kh[:, h // c["G"], :] @ qh[h]).max() for h in range(Hq)]) * scale
                bar = 1e-3 + 2.0**-12 * mag
            assert np.all(np.abs(lse[b, i] - ref["lse"][i]) <= bar), (b, i)


N_KIVI = 16


@pytest.mark.parametrize("case", range(N_KIVI))
def test_kivi_option_combinations(case):
    """KIVI caches: code width, group, verification positions, partitions,
    lengths across the window and group boundaries, shuffled pages and append
    plans (one bulk call, or bulk + one-token steps + rest); state bit-exact and
    outputs against the oracle."""
    from tests.test_gpu_kivi import check_state
    rng = np.random.default_rng(5000 + case)
    bits = int(rng.choice([4, 2]))
    n_kv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    QL = int(rng.choice([1, 1, 2, 4]))
    while G * QL > 16:
        QL //= 2
    B = int(rng.integers(1, 5))
    lens = rng.integers(1, 700, size=B)
    part = int(rng.choice([0, 0, 1, 3]))
    say("kivi", case, dict(bits=bits, n_kv=n_kv, G=G, QL=QL, lens=lens.tolist(), part=part))
    d = dict(synthetic.WORKLOADS["kivi" if bits == 4 else "kivi2"].__dict__)
    d.update(batch=B, num_q_heads=n_kv * G, num_kv_heads=n_kv, context=int(lens.max()), seed=70 + case)
    w = synthetic.Workload(**d)
    plan = None if rng.integers(2) else [lens]
    bt = H.build_kivi(w, lens, plan=plan, shuffle=bool(rng.integers(2)))
    Hq, dh = w.num_q_heads, w.head_dim
    scale = dh ** -0.5
    q = synthetic.gen_q(w, "cuda", batch=B * QL).reshape(B, QL, Hq, dh).contiguous()
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, QL, Hq, bt.max_ctx, part), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, QL, Hq, dh), float("nan"), device="cuda")
    lse = torch.full((B, QL, Hq), float("nan"), device="cuda")
    kvq.verify_attention(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, scale, ws, out, lse, part)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qc = synthetic.gen_q(w, "cpu", batch=B * QL).reshape(B, QL, Hq, dh)
    for b in range(B):
        ref = H.kivi_oracle_seq(bt, b)
        check_state(bt, b, ref)
        T = int(lens[b])
        for i in range(QL):
            n_vis = T - QL + 1 + i
            if n_vis <= 0:
                assert not out[b, i].any() and np.all(np.isneginf(lse[b, i])), (b, i)
                continue
            qi = O.bf16_value(H.u16(qc[b, i])).astype(np.float64)
            o_ref, l_ref = O.attention(qi, ref["k_hat"][:n_vis], ref["v_hat"][:n_vis], scale)
            ok, mabs, mrel = H.allclose_report(out[b, i], o_ref, ATOL, RTOL)
            assert ok, f"seq {b} position {i}: max abs {mabs:.3e} max rel {mrel:.3e}"
            assert np.abs(lse[b, i] - l_ref).max() <= 1e-3, (b, i)
