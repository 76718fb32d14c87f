"""Benchmark of the paged FP8 / INT8 KV-cache decode step on one MI355X.

One step = the whole hot path for one decode token per sequence:
  kvq_append (quantize the new K/V row into its page slot)
  + split-K decode attention over the quantized paged cache
  + log-sum-exp merge of the partial results.
Inputs are seeded synthetic tensors (``synthetic.py``) with the workload's
shapes, resident in HBM before timing starts.

    python bench.py [--config llama70b] [--steps 100] [--warmup 10]

Prints one JSON line.  ``value`` is algorithmic bytes of the step / step time
(GB/s); ``roofline`` reports the split-K decode kernel (the dominant one)
against the 8 TB/s HBM peak with per-launch HIP-event timing; ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# decoder layers of the models whose attention shape (query heads, KV heads)
# the workloads take: Llama-3-8B (32 / 8, 32 layers), Llama-3-70B (64 / 8, 80)
MODEL_LAYERS = {(32, 8): 32, (64, 8): 80}
DECODE_SRC = os.path.join(ROOT, "quantized_kv_cache_08_amd", "csrc", "decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama70b",
                    choices=["tiny", "llama8b", "llama70b", "mixed", "kivi", "kivi2", "verify", "e5m2", "static", "fp8qk",
                             "fp8attn"])
    ap.add_argument("--replicas", type=int, default=0, help="cache copies rotated per step (0 = auto)")
    ap.add_argument("--partition-pages", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="time the whole step as replays of one HIP graph per cache replica (slower than "
                         "eager launches on ROCm 7)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="rough CPU work budget for the oracle sample")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# Sources each split kernel is built from: its own file plus the shared
# headers and the host layer that sizes its launch.
_SHARED_SRC = ("splitk.h", "kvq_device.h", "kvq_internal.h", "kvq_api.cpp")
_KERNEL_SRC = {"decode": ("decode.hip",) + _SHARED_SRC, "kivi": ("kivi.hip", "decode.hip") + _SHARED_SRC}


def source_hash(config: str = "llama8b") -> str:
    """Hash of the sources of the workload's split kernel (the KIVI path also
    launches the reduce kernel of decode.hip), so that recorded counters are
    used only while that kernel is unchanged."""
    import synthetic
    kind = "kivi" if synthetic.WORKLOADS[config].kivi_bits else "decode"
    h = hashlib.sha256()
    d = os.path.dirname(DECODE_SRC)
    for f in sorted(_KERNEL_SRC[kind]):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def kivi_quantized(w, lens: np.ndarray) -> np.ndarray:
    """Tokens per sequence held as INT4 groups: 32 * floor(max(0, n - residual) / 32)."""
    over = np.maximum(0, np.asarray(lens, dtype=np.int64) - w.resid)
    return (over // w.page_size) * w.page_size


def step_bytes(w, lens: np.ndarray):
    """Algorithmic bytes of one step, split by kernel."""
    n_kv, d, Hq = w.num_kv_heads, w.head_dim, w.num_q_heads
    tokens = int(lens.sum())
    B = len(lens)
    QL = w.q_len                                       # query positions per sequence
    if w.kivi_bits:
        codes = w.page_size * d * w.kivi_bits // 8         # INT4 / INT2 page records (codes + bf16 s, z)
        rk, rv = codes + 4 * d, codes + 4 * w.page_size
        nq = kivi_quantized(w, lens)
        pages = int((nq // w.page_size).sum())
        window = (tokens - int(nq.sum())) * n_kv * d * 2 * 2  # fp16 K and V rows
        kv = pages * n_kv * (rk + rv) + window
        split = kv + pages * 4 + B * Hq * d * 2
        # one new token per sequence: bf16 in, fp16 window row out; a group flush
        # (32 fp16 window rows in, one K and one V record out) when it completes one
        flushes = int((kivi_quantized(w, lens) > kivi_quantized(w, lens - 1)).sum())
        append = B * n_kv * d * 2 * 2 * 2 + flushes * n_kv * (32 * d * 2 * 2 + rk + rv) + B * 8
    else:
        # bf16 scale (+ bf16 zero-point) per (token, head); none with static scales
        meta = 0 if w.scale_mode != 2 else (4 if w.dtype == "int8" else 2)
        pages = int(((lens + w.page_size - 1) // w.page_size).sum())
        kv = tokens * n_kv * 2 * (d + meta)
        split = kv + pages * 4 + B * QL * Hq * d * 2   # K/V codes+scales, block-table entries, q
        append = QL * (B * n_kv * 2 * (d * 2 + d + meta) + B * 4)
    reduce = B * QL * Hq * d * 4                       # out (fp32)
    return dict(kv=kv, split=split, reduce=reduce, append=append, total=split + reduce + append,
                tokens=tokens, pages=pages)


def slots_for(layout, b: int, pos0: int, n: int, ps: int):
    import torch
    pos = np.arange(pos0, pos0 + n, dtype=np.int64)
    pages = layout.block_table[b, pos // ps].astype(np.int64)
    return torch.from_numpy((pages * ps + pos % ps).astype(np.int32)).cuda()


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(w, budget_s: float):
    """The CPU oracle (as it stands) on a bounded sample of the workload:
    quantize-on-store of whole sequences plus fp64 decode attention over
    them.  Sequences are generated in order until about half the budget has
    gone to generation and oracle time together; the oracle then cycles over
    the held sequences until about ``budget_s`` seconds of oracle time."""
    import torch
    import synthetic
    from oracle import oracle as O

    lens = synthetic.seq_lens(w)
    kivi = w.kivi_bits > 0
    if kivi:
        # a 16384-token prefix of each sequence keeps one pass to a few seconds
        lens = np.minimum(lens, 16384)
    dt = {"fp8": O.FP8, "e5m2": O.E5M2, "int8": O.INT8, "kivi4": None, "kivi2": None}[w.dtype]
    QL = w.q_len
    static_kv = None
    if w.scale_mode != 2:
        ss = synthetic.static_scales(w).view(torch.int16).numpy().view(np.uint16)
        static_kv = (ss[0], ss[1])
    q_all = synthetic.gen_q(w, "cpu", batch=len(lens) * QL)
    if QL > 1:
        q_all = q_all.reshape(len(lens), QL, w.num_q_heads, w.head_dim)
    scale = 1.0 / math.sqrt(w.head_dim)

    def run_oracle(qb, kb, vb):
        """One sequence through the oracle: store-time quantization, then fp64
        attention over the dequantized cache; returns the two times."""
        t0 = time.perf_counter()
        if not kivi:
            res = O.quantized_cache(kb, vb, dt, w.scale_mode, static_kv)
            kh, vh = res["k_hat"], res["v_hat"]
        else:
            k16, v16 = O.bf16_to_f16_bits(kb), O.bf16_to_f16_bits(vb)
            kh = np.zeros((kb.shape[0], w.num_kv_heads, w.head_dim))
            vh = np.zeros_like(kh)
            for h in range(w.num_kv_heads):
                st = O.kivi_stream(k16[:, h], v16[:, h], w.resid, w.page_size, w.kivi_bits)
                kh[:, h], vh[:, h] = O.kivi_dequant(st, w.page_size)
        t1 = time.perf_counter()
        q = O.fp8_query(qb) if w.fp8_qk else O.bf16_value(qb).astype(np.float64)
        if w.fp8_pv:
            O.attention_fp8pv(q, kh, O.v_code_values(dt, res["v_codes"]), O.bf16_value(res["v_scale"]), scale)
        elif QL == 1:
            O.attention(q, kh, vh, scale)
        else:
            T = kh.shape[0]
            for i in range(QL):
                n_vis = max(0, T - QL + 1 + i)
                O.attention(q[i], kh[:n_vis], vh[:n_vis], scale)
        return t1 - t0, time.perf_counter() - t1

    held = []
    t_total, t_quant, t_attn, done = 0.0, 0.0, 0.0, []
    wall0 = time.perf_counter()
    i = 0
    while t_total < budget_s and len(done) < 100000:
        grow = (len(held) < len(lens) and time.perf_counter() - wall0 < budget_s / 2) or not held
        if grow:
            b = len(held)
            T = int(lens[b])
            k, v = synthetic.gen_kv(w, b, 0, T, "cpu")
            kb = k.view(torch.int16).numpy().view(np.uint16)
            vb = v.view(torch.int16).numpy().view(np.uint16)
            qb = q_all[b].contiguous().view(torch.int16).numpy().view(np.uint16)
            held.append((T, qb, kb, vb))
            cur = held[-1]
        else:
            cur = held[i % len(held)]
            i += 1
        T, qb, kb, vb = cur
        tq, ta = run_oracle(qb, kb, vb)
        t_quant += tq
        t_attn += ta
        t_total += tq + ta
        done.append(T)
        if len(done) % 16 == 1:
            print(f"[cpu_baseline] {len(done)} passes, {t_total:.1f} s oracle time", file=sys.stderr, flush=True)
    sl = np.array(done)
    by = step_bytes(w, sl)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(by["kv"] / t_total / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(done)} sequence passes over the first {len(held)} of {len(lens)} sequences "
                      + ("(16384-token prefixes) " if kivi else "") +
                      f"({int(sl.sum())} tokens): quantize-on-store of their K/V plus fp64 attention"
                      + (f" of {QL} causal positions each" if QL > 1 else "") + ", "
                      f"{t_total:.1f} s; value = their K/V code+scale bytes / time",
            "tokens_per_s": round(len(done) / t_total, 4),
            "quantize_s": round(t_quant, 3), "attention_s": round(t_attn, 3)}


# (workgroups per CU, 16-byte loads in flight per thread) tried by the read
# probe: 16 to 48 KiB in flight per CU, where a streaming read on this part
# peaks (about 24 KiB)
READ_SHAPES = ((1, 4), (1, 6), (2, 2), (2, 3), (2, 4), (3, 2), (4, 1), (4, 2), (3, 4))


def attainable_read(nbytes: int, launches: int = 20) -> dict:
    """A plain streaming read (kvq_read_probe) of as many bytes as the split
    kernel reads per launch, from two buffers used in turn (so that each launch
    reads data the previous one did not leave in the last-level cache), timed
    back to back between two events; the best of the launch shapes in
    READ_SHAPES."""
    import torch
    from quantized_kv_cache_08_amd import testing as KT
    n = max(16, nbytes // 16 * 16)
    bufs = [torch.full((n,), i + 1, dtype=torch.uint8, device="cuda") for i in range(2)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for bpc, lpt in READ_SHAPES:
        for i in range(4):
            KT.read_probe(bufs[i % 2], sink, bpc, lpt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(launches):
            KT.read_probe(bufs[i % 2], sink, bpc, lpt)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        gbs = n / (us * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "us": round(us, 2), "blocks_per_cu": bpc, "loads_per_thread": lpt}
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "plain streaming read of the split kernel's byte count (kvq_read_probe)", "bytes": n,
            "frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4), **best}


def oracle_threads(n: int) -> int:
    """Set the oracle's OpenMP thread count; returns the previous one."""
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    prev = gomp.omp_get_max_threads()
    gomp.omp_set_num_threads(int(n))
    return prev


def read_traffic(config: str):
    """HBM bytes per split launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources."""
    f = os.path.join(ROOT, "profiles", f"split_kernel_{config}_traffic.txt")
    if not os.path.exists(f):
        return None
    kv = {}
    for line in open(f):
        if ":" in line:
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_hash") != source_hash(config):
        return None
    try:
        return int(float(kv["bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU build: this benchmark runs on one GPU only",
                          "requested_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import quantized_kv_cache_08_amd as kvq
    import synthetic

    if args.copy_calib_mib:
        copy_calibration(args.copy_calib_mib)
        return

    torch.cuda.set_device(0)
    w = synthetic.WORKLOADS[args.config]
    lens = synthetic.seq_lens(w)
    B, Hq, d = len(lens), w.num_q_heads, w.head_dim
    by = step_bytes(w, lens)
    reps = args.replicas or (2 if by["kv"] < (1 << 30) else 1)

    # each cache replica holds the context minus the newest token (pages laid
    # out for the full length); every step appends that token, then decodes.
    # A verification workload (q_len > 1) holds all but the q_len newest
    # positions, appends those and scores them causally.
    kivi = w.kivi_bits > 0
    QL = w.q_len
    full_layout = synthetic.page_layout(w, lens)
    bt_dev = torch.from_numpy(full_layout.block_table).cuda()
    caches = []
    for r in range(reps):
        if kivi:
            cache = kvq.Cache(kvq.KVQ_INT2_KIVI if w.kivi_bits == 2 else kvq.KVQ_INT4_KIVI, full_layout.num_pages, w.num_kv_heads, w.page_size, d,
                              max_seqs=B, residual=w.resid)
            held = np.zeros(B, dtype=np.int64)
            target = lens - 1
            while (held < target).any():
                step_n = np.minimum(target - held, 1 << 14)
                ks, vs = [], []
                for b in range(B):
                    if step_n[b]:
                        k, v = synthetic.gen_kv(w, b, int(held[b]), int(step_n[b]), "cuda")
                        ks.append(k)
                        vs.append(v)
                offs = torch.from_numpy(np.concatenate([[0], np.cumsum(step_n)]).astype(np.int32)).cuda()
                kvq.kivi_append(cache, torch.cat(ks), torch.cat(vs), offs,
                                torch.from_numpy(held.astype(np.int32)).cuda(), bt_dev, int(step_n.max()))
                held += step_n
        else:
            code = {"fp8": kvq.KVQ_FP8_E4M3, "e5m2": kvq.KVQ_FP8_E5M2, "int8": kvq.KVQ_INT8_ASYM}[w.dtype]
            ss = synthetic.static_scales(w).cuda() if w.scale_mode != 2 else None
            flags = (kvq.KVQ_ATTN_FP8_QK if w.fp8_qk else 0) | (kvq.KVQ_ATTN_FP8_PV if w.fp8_pv else 0)
            cache = kvq.Cache(code, full_layout.num_pages, w.num_kv_heads, w.page_size, d, w.scale_mode, ss,
                              attn_flags=flags)
            for b, n in enumerate(lens):
                m = int(n) - QL
                for p0 in range(0, m, 1 << 16):
                    mm = min(1 << 16, m - p0)
                    k, v = synthetic.gen_kv(w, b, p0, mm, "cuda")
                    kvq.append(cache, k, v, slots_for(full_layout, b, p0, mm, w.page_size))
        caches.append(cache)
        print(f"[bench] cache replica {r} filled", file=sys.stderr, flush=True)
    cl_dev = torch.from_numpy(lens.astype(np.int32)).cuda()
    cl_before = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    new_offs = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    if QL == 1:
        q = synthetic.gen_q(w, "cuda")
    else:
        q = synthetic.gen_q(w, "cuda", batch=B * QL).reshape(B, QL, Hq, d)
    knew = torch.empty(B * QL, w.num_kv_heads, d, dtype=torch.bfloat16, device="cuda")
    vnew = torch.empty_like(knew)
    for b in range(B):
        kk, vv = synthetic.gen_new_kv(w, b, QL, "cuda")
        knew[b * QL:(b + 1) * QL], vnew[b * QL:(b + 1) * QL] = kk, vv
    pos = (lens[:, None] - QL + np.arange(QL)[None, :]).reshape(-1)
    seq = np.repeat(np.arange(B), QL)
    slot = (full_layout.block_table[seq, pos // w.page_size].astype(np.int64) * w.page_size
            + pos % w.page_size).astype(np.int32)
    slot_dev = torch.from_numpy(slot).cuda()
    max_ctx = int(lens.max())
    if QL == 1:
        ws_bytes = kvq.decode_workspace_bytes(caches[0], B, Hq, max_ctx, args.partition_pages)
        out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    else:
        ws_bytes = kvq.verify_workspace_bytes(caches[0], B, QL, Hq, max_ctx, args.partition_pages)
        out = torch.empty(B, QL, Hq, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(d)
    torch.cuda.synchronize()

    def split(c):
        if QL == 1:
            kvq.decode_split(c, q, bt_dev, cl_dev, max_ctx, scale, ws, out, None, args.partition_pages)
        else:
            kvq.verify_split(c, q, bt_dev, cl_dev, max_ctx, scale, ws, out, None, args.partition_pages)

    def reduce(c):
        if QL == 1:
            kvq.decode_reduce(c, B, Hq, max_ctx, ws, out, None, args.partition_pages)
        else:
            kvq.verify_reduce(c, B, QL, Hq, max_ctx, ws, out, None, args.partition_pages)

    def step(i, ev=None):
        c = caches[i % reps]
        if ev is not None:
            ev[0].record()
        if kivi:
            kvq.kivi_append(c, knew, vnew, new_offs, cl_before, bt_dev, 1)
        else:
            kvq.append(c, knew, vnew, slot_dev)
        if ev is not None:
            ev[1].record()
        split(c)
        if ev is not None:
            ev[2].record()
        reduce(c)
        if ev is not None:
            ev[3].record()

    # per-kernel times: a pass of eager steps with an event between the launches
    # (the events cost a few microseconds per step, so the whole-step time is
    # taken in a second pass without them)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()

    # mean launch duration of each kernel: K back-to-back launches of that kernel
    # alone between two events (a single launch between events also counts its
    # dispatch latency); the split launches alternate cache replicas like the steps
    def back_to_back(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn(0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def app(i):
        if kivi:
            kvq.kivi_append(caches[i % reps], knew, vnew, new_offs, cl_before, bt_dev, 1)
        else:
            kvq.append(caches[i % reps], knew, vnew, slot_dev)
    mean_app = back_to_back(app)
    mean_split = back_to_back(lambda i: split(caches[i % reps]))
    mean_red = back_to_back(lambda i: reduce(caches[i % reps]))

    # whole-step time: the same steps as eager launches on the stream, or with
    # --graph as replays of one HIP graph per cache replica
    if not args.graph:
        run = step
    else:
        graphs = []
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        run = lambda i: graphs[i % reps].replay()     # noqa: E731
    for i in range(args.warmup):
        run(i)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        run(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    t_split = np.array([e[1].elapsed_time(e[2]) for e in evs])

    value = by["total"] / (ms_step * 1e-3) / 1e9
    split_gbs = by["split"] / (mean_split * 1e-3) / 1e9
    attn_ms = mean_split + mean_red
    kv_gbs = (by["split"] + by["reduce"]) / (attn_ms * 1e-3) / 1e9

    traffic = read_traffic(args.config)
    attain = attainable_read(by["split"])

    res = {
        "metric": "paged FP8/INT8 decode-attn KV GB/s (% of HBM peak) + tokens/s at 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"fp8": "fp8_e4m3", "e5m2": "fp8_e5m2", "int8": "u8", "kivi4": "u4", "kivi2": "u2"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "batch": B, "num_q_heads": Hq,
                   "num_kv_heads": w.num_kv_heads, "head_dim": d, "page_size": w.page_size,
                   "context_tokens": by["tokens"], "max_context": max_ctx, "cache_replicas": reps,
                   "partition_pages": args.partition_pages or "auto", "positions_per_seq": QL,
                   "scale_mode": {2: "per_token_head", 1: "static_per_head", 0: "static_per_tensor"}[w.scale_mode],
                   "qk": "fp8_domain (query in E4M3)" if w.fp8_qk else "bf16 query",
                   "pv": "fp8_domain (probabilities in E4M3, 32-token power-of-two block scales)" if w.fp8_pv
                         else "bf16 hi + lo probabilities",
                   "step_launch": "hip_graph" if args.graph else "eager"},
        "tokens_per_s": round(B * QL / (ms_step * 1e-3), 1),
        # attention-only extrapolation to a whole model of this layer's shape:
        # every layer runs the same step, nothing else of the model is timed
        "tokens_per_s_attention_only_model": (
            None if not MODEL_LAYERS.get((Hq, w.num_kv_heads)) else
            {"layers": MODEL_LAYERS[(Hq, w.num_kv_heads)],
             "value": round(B * QL / (ms_step * 1e-3 * MODEL_LAYERS[(Hq, w.num_kv_heads)]), 1)}),
        # split + reduce bytes over both kernels' back-to-back means (the reduce
        # mean is dispatch-bound); the split kernel alone is `roofline`
        "split_plus_reduce_kv_gbs": round(kv_gbs, 2),
        "split_plus_reduce_pct_of_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        # means: back-to-back launches; p50 / p95: single launches between events
        # (these include each launch's dispatch latency)
        "kernel_ms": {"append": round(float(mean_app), 5), "split": round(float(mean_split), 5),
                      "reduce": round(float(mean_red), 5),
                      "split_p50": round(float(np.median(t_split)), 5),
                      "split_p95": round(float(np.percentile(t_split, 95)), 5),
                      "split_single_launch_mean": round(float(t_split.mean()), 5)},
        "algorithmic_bytes": {k: by[k] for k in ("kv", "split", "reduce", "append", "total")},
        "roofline": {"bound": "hbm", "kernel": "split_kernel (paged split-K decode attention)",
                     "achieved": round(split_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "source_hash": source_hash(args.config),
        "attainable": dict(attain, split_frac_of_attainable=round(split_gbs / attain["gbs"], 4)),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        # the same oracle on one host thread, a shorter sample
        threads = oracle_threads(1)
        one = cpu_baseline(w, max(2.0, args.cpu_seconds / 3))
        oracle_threads(threads)
        res["cpu_baseline"]["one_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                                             "sample": one["sample"]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
