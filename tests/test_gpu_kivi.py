"""GPU parity of the KIVI-style path (kvq_kivi_append + kvq_kivi_decode_attention on
a KVQ_INT4_KIVI or KVQ_INT2_KIVI cache) against the CPU oracle.

Quantized bytes (4-bit or 2-bit codes, per-channel K and per-token V BF16
scales and zero-points) and the fp16 window rows must match bit for bit;
attention must satisfy |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise
against fp64 attention over the oracle's own dequantized tokens plus fp16
window.  Every case runs at both code widths.
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
from tests import kvq_harness as H  # noqa: E402
from oracle import oracle as O  # noqa: E402

ATOL, RTOL = 2e-3, 1e-2
LSE_ATOL = 1e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


BITS = pytest.mark.parametrize("bits", [4, 2])


def small(bits=4, **kw) -> synthetic.Workload:
    w = synthetic.WORKLOADS["kivi" if bits == 4 else "kivi2"]
    d = dict(w.__dict__)
    d.update(dict(batch=3, num_q_heads=8, num_kv_heads=2, context=1024))
    d.update(kw)
    return synthetic.Workload(**d)


def check_state(bt, b, ref):
    got = H.kivi_read_seq(bt, b)
    for h, (g, r) in enumerate(zip(got, ref["heads"])):
        assert g["nq"] == r["nq"]
        for key in ("k_codes", "k_s", "k_z", "v_codes", "v_s", "v_z", "k_res", "v_res"):
            a, e = np.asarray(g[key]), np.asarray(r[key])
            assert a.shape == e.shape, (key, a.shape, e.shape)
            if not np.array_equal(a, e):
                idx = np.argwhere(a != e)[0]
                raise AssertionError(f"seq {b} head {h} {key} differs at {tuple(idx)}: {a[tuple(idx)]} vs {e[tuple(idx)]}")


def check_out(bt, out, lse, b, ref):
    """Outputs within 2e-3 + 1e-2 |ref| and lse within 1e-3 of the oracle;
    returns (max abs, max rel, max lse) deviation."""
    ok, mabs, mrel = H.allclose_report(out[b].cpu().numpy(), ref["out"], ATOL, RTOL)
    assert ok, f"seq {b}: max abs {mabs:.3e} max rel {mrel:.3e}"
    dl = np.abs(lse[b].cpu().numpy().astype(np.float64) - ref["lse"])
    assert dl.max() <= LSE_ATOL, f"seq {b}: lse diff {dl.max():.3e}"
    return mabs, mrel, float(dl.max())


@BITS
def test_kivi_append_and_decode_small(bits):
    """Window-only, one group, several groups; groups flushed from the window,
    from new rows and from both (bulk call, one-token steps, remainder)."""
    w = small(bits)
    lens = np.array([100, 200, 333])
    say("kivi small build", bits)
    bt = H.build_kivi(w, lens)
    out, lse = H.run_decode_kivi(bt)
    for b in range(len(lens)):
        say("kivi small check seq", b)
        ref = H.kivi_oracle_seq(bt, b)
        check_state(bt, b, ref)
        check_out(bt, out, lse, b, ref)


@BITS
def test_kivi_group_boundaries_one_token_at_a_time(bits):
    """Appending one token per call across the 160/192-token boundaries flushes a
    group from the window exactly when the window would exceed 128 + 31 tokens."""
    w = small(bits, batch=2)
    lens = np.array([161, 197])
    plan = [np.array([120, 120])] + [np.array([1 if 120 + i < n else 0 for n in lens]) for i in range(80)]
    say("kivi one-token build", bits)
    bt = H.build_kivi(w, lens, plan=plan)
    out, lse = H.run_decode_kivi(bt)
    for b in range(2):
        ref = H.kivi_oracle_seq(bt, b)
        check_state(bt, b, ref)
        check_out(bt, out, lse, b, ref)


@BITS
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_kivi_gqa_group_sizes(G, bits):
    w = small(bits, batch=2, num_q_heads=2 * G, num_kv_heads=2)
    lens = np.array([290, 77])
    say("kivi gqa", G, bits)
    bt = H.build_kivi(w, lens)
    out, lse = H.run_decode_kivi(bt)
    for b in range(2):
        check_out(bt, out, lse, b, H.kivi_oracle_seq(bt, b))


@BITS
def test_kivi_partition_sweep_and_shuffled_pages(bits):
    w = small(bits, batch=4, num_q_heads=16, num_kv_heads=2)
    lens = np.array([1000, 1, 450, 161])
    say("kivi partitions build", bits)
    bt = H.build_kivi(w, lens, shuffle=True)
    refs = [H.kivi_oracle_seq(bt, b) for b in range(len(lens))]
    outs = []
    for part in (0, 1, 2, 3, 7, 64):
        say("kivi partitions decode", part)
        out, lse = H.run_decode_kivi(bt, part)
        for b in range(len(lens)):
            check_out(bt, out, lse, b, refs[b])
        outs.append(out.cpu())
    # V codes enter the MFMA as 128 + n and the offset is removed at the end, so
    # fp32 rounding of the accumulator is amplified by about (128 + 7.5) / 7.5
    # (4 bits; (128 + 1.5) / 1.5 at 2 bits, with steps 5x larger); different
    # partitionings round differently by up to ~1e-4 (the oracle bar above is
    # 2e-3 + 1e-2 |ref|)
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], atol=5e-4, rtol=1e-4)


@BITS
def test_kivi_context_length_one_is_exact(bits):
    """One token, still in the fp16 window: the output is its fp16 value row exactly."""
    w = small(bits, batch=2)
    bt = H.build_kivi(w, np.array([1, 1]))
    out, lse = H.run_decode_kivi(bt)
    for b in range(2):
        ref = H.kivi_oracle_seq(bt, b)
        vrow = np.repeat(ref["v_hat"][0], w.group_size, axis=0)
        assert np.array_equal(out[b].cpu().numpy().astype(np.float64), vrow)


@BITS
def test_kivi_full_size(bits):
    """B 4, 64 q / 8 KV heads, context 131072 (130944 quantized tokens + 128
    fp16).  Every sequence: the whole state (codes, scales, zero-points, window
    rows) bit for bit, and the outputs of two plans against the oracle: the
    automatic one (64 segments per item, one range per resident wave) and one
    segment per item (4096 pages through a single running state, the longest
    fp32 accumulation the code offset of 128 can amplify).  The largest
    deviations are printed ([margin] lines)."""
    w = synthetic.WORKLOADS["kivi" if bits == 4 else "kivi2"]
    say("kivi full build", bits)
    bt = H.build_kivi(w, plan=[synthetic.seq_lens(w) - 5, np.ones(w.batch, dtype=np.int64) * 5])
    say("kivi full decode")
    plans = {"auto": H.run_decode_kivi(bt), "one segment per item": H.run_decode_kivi(bt, 4096)}
    worst = {k: [0.0, 0.0, 0.0] for k in plans}
    for b in range(w.batch):
        say("kivi full check seq", b)
        ref = H.kivi_oracle_seq(bt, b)
        check_state(bt, b, ref)
        for name, (out, lse) in plans.items():
            got = check_out(bt, out, lse, b, ref)
            worst[name] = [max(a, g) for a, g in zip(worst[name], got)]
        del ref
    for name, (mabs, mrel, mlse) in worst.items():
        say(f"[margin] KIVI {bits}-bit full size, {name}: max abs {mabs:.3e}, max rel {mrel:.3e}, "
            f"max lse {mlse:.3e}")


@BITS
def test_kivi_decode_step_as_hip_graph_matches_eager(bits):
    """One-token KIVI append (re-appending each sequence's last token, which
    completes a group for the first length) and decode, captured as a HIP graph:
    every replay, with eager work in between, reproduces the eager outputs."""
    from tests.test_gpu_parity import _graph_replays_match
    w = small(bits, batch=2, num_q_heads=16, num_kv_heads=2)
    lens = np.array([160, 300])
    say("kivi graph step build", bits)
    bt = H.build_kivi(w, lens)
    B, Hq, d = bt.q.shape[0], bt.q.shape[1], bt.w.head_dim
    rows = [synthetic.gen_kv(w, b, int(lens[b]) - 1, 1, "cuda") for b in range(B)]
    knew = torch.cat([r[0] for r in rows]).contiguous()
    vnew = torch.cat([r[1] for r in rows]).contiguous()
    offs = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    before = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    ws = torch.empty(kvq.decode_workspace_bytes(bt.cache, B, Hq, bt.max_ctx, 2), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    out = torch.empty(B, Hq, d, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    out2 = torch.empty_like(out)
    scale = 1.0 / np.sqrt(d)

    def step():
        kvq.kivi_append(bt.cache, knew, vnew, offs, before, bt.block_table, 1)
        kvq.decode_split(bt.cache, bt.q, bt.block_table, bt.context_lens, bt.max_ctx, scale, ws, out, lse, 2)
        kvq.decode_reduce(bt.cache, B, Hq, bt.max_ctx, ws, out, lse, 2)

    def other():
        kvq.kivi_decode_attention(bt.cache, bt.q, bt.block_table, bt.context_lens, bt.max_ctx, scale, ws2, out2, None, 2)

    _graph_replays_match(step, [out, lse], other)
    for b in range(B):
        check_out(bt, out, lse, b, H.kivi_oracle_seq(bt, b))


@BITS
@pytest.mark.parametrize("G,q_len", [(2, 4), (4, 4), (8, 2)])
def test_kivi_verification_pass(bits, G, q_len):
    """The q_len newest positions scored causally over a KIVI cache (rows per
    KV head G q_len = 8 shares lanes, 16 does not): position i sees the first
    len - q_len + 1 + i tokens; a position that sees none gives out 0, lse -inf."""
    from oracle import oracle as O
    w = small(bits, batch=4, num_q_heads=2 * G, num_kv_heads=2)
    lens = np.array([2, 100, 161, 300])
    say("kivi verify", bits, G, q_len)
    bt = H.build_kivi(w, lens)
    B, Hq, d = len(lens), w.num_q_heads, w.head_dim
    q = synthetic.gen_q(w, "cuda", batch=B * q_len).reshape(B, q_len, Hq, d)
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, q_len, Hq, bt.max_ctx), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, q_len, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, q_len, Hq), float("nan"), device="cuda")
    kvq.verify_attention(bt.cache, q, bt.block_table, bt.context_lens, bt.max_ctx, d ** -0.5, ws, out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qc = synthetic.gen_q(w, "cpu", batch=B * q_len).reshape(B, q_len, Hq, d)
    for b in range(B):
        ref = H.kivi_oracle_seq(bt, b)
        T = int(lens[b])
        for i in range(q_len):
            n_vis = T - q_len + 1 + i
            if n_vis <= 0:
                assert not out[b, i].any() and np.all(np.isneginf(lse[b, i])), (b, i)
                continue
            qi = O.bf16_value(H.u16(qc[b, i])).astype(np.float64)
            o_ref, l_ref = O.attention(qi, ref["k_hat"][:n_vis], ref["v_hat"][:n_vis], d ** -0.5)
            ok, mabs, mrel = H.allclose_report(out[b, i], o_ref, ATOL, RTOL)
            assert ok, f"seq {b} position {i}: max abs {mabs:.3e} max rel {mrel:.3e}"
            assert np.abs(lse[b, i] - l_ref).max() <= LSE_ATOL, (b, i)


@BITS
def test_kivi_verify_one_position_is_decode_bit_for_bit(bits):
    w = small(bits, batch=3, num_q_heads=8, num_kv_heads=2)
    bt = H.build_kivi(w, np.array([1, 170, 333]))
    out_d, lse_d = H.run_decode_kivi(bt)
    B, Hq, d = 3, 8, w.head_dim
    ws = torch.zeros(kvq.verify_workspace_bytes(bt.cache, B, 1, Hq, bt.max_ctx), dtype=torch.uint8, device="cuda")
    out = torch.full((B, 1, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, 1, Hq), float("nan"), device="cuda")
    kvq.verify_attention(bt.cache, bt.q.reshape(B, 1, Hq, d).contiguous(), bt.block_table, bt.context_lens,
                         bt.max_ctx, d ** -0.5, ws, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0], out_d) and torch.equal(lse[:, 0], lse_d)


@BITS
@pytest.mark.parametrize("resid", [0, 32])
def test_kivi_short_windows(bits, resid):
    """The window rule with other residual sizes: residual 0 keeps only the
    partial newest group in fp16 (n_q = 32 floor(n / 32)), residual 32 up to 63
    tokens; state bit-exact, attention against the oracle."""
    w = small(bits, batch=3, resid=resid)
    lens = np.array([31, 64, 250])
    say("kivi residual", resid, bits)
    bt = H.build_kivi(w, lens)
    out, lse = H.run_decode_kivi(bt)
    for b in range(len(lens)):
        ref = H.kivi_oracle_seq(bt, b)
        check_state(bt, b, ref)
        check_out(bt, out, lse, b, ref)


@BITS
@pytest.mark.parametrize("G", [8, 16])
def test_kivi_rescales_of_the_running_state(bits, G):
    """At softmax scale 0.25 the chunk maxima of a head rise past the kernel's
    rescale headroom (2^8) many times within a sequence (counted below on the
    oracle's scores), so the running state is rescaled with non-zero sums; with
    query groups up to 8 that includes the accumulator rows holding the
    lo-part products.  One segment per sequence keeps every jump inside one
    running state."""
    w = small(bits, batch=2, num_q_heads=2 * G, num_kv_heads=2)
    lens = np.array([700, 1000])
    scale = 0.25
    bt = H.build_kivi(w, lens)
    out, lse = H.run_decode_kivi(bt, partition_pages=1024, softmax_scale=scale)
    jumps = 0
    for b in range(len(lens)):
        ref = H.kivi_oracle_seq(bt, b, softmax_scale=scale)
        q = O.bf16_value(H.u16(synthetic.gen_q(w, "cpu", batch=len(lens))[b])).astype(np.float64)
        for hq in range(w.num_q_heads):
            s = ref["k_hat"][:, hq // G] @ q[hq] * (scale / np.log(2.0))
            m = s[:32].max()
            for c in range(32, int(lens[b]), 32):
                mx = s[c:c + 32].max()
                jumps += int(mx > m + 8.0)
                m = max(m, mx)
        check_state(bt, b, ref)
        check_out(bt, out, lse, b, ref)
    assert jumps >= 10, jumps
