// splitk.h -- work distribution shared by the split-K decode kernels.
//
// Flash-decoding over context partitions, balanced across the whole batch:
// each (sequence, KV head) is an "item" of pages (32-token chunks for the
// KIVI window path, which counts its fp16 tail as trailing chunks).  For each
// KV head the items of all sequences are laid end to end, and that head's
// page space is cut into equal ranges, the same cut for every head, one range
// per resident wave.  A wave walks its range item by item and calls the
// segment processor once per (item, sub-range).  A segment that covers a
// whole item writes the final result; otherwise it writes partial results that
// the reduce kernel merges with log-sum-exp weights.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"
#include "split_plan.h"

namespace kvq {

// Merge of the n partial results of one (sequence, query head) row:
//   L = max_i lse_i,  w_i = 2^(lse_i - L),  out = sum_i w_i o_i / sum_i w_i,
//   lse = (L + log2 sum_i w_i) * ln 2,
// computed online over groups of 8 partials.  Called by all 64 lanes of a
// wave; each lane merges channels 2 lane, 2 lane + 1.  Partial i has lse
// pl[i * stride] and row po[i * stride * 128 + ..].  All loads of a group (8
// lse values and 8 partial rows, every lane reading the same lse words) are
// issued before any is used, so that a merge of up to 8 partials costs one
// memory round trip.
__device__ __forceinline__ void merge_row(const float* pl, const float* po, long long stride, int n,
                                          float* out, float* lse, int lane) {
    float m = -INFINITY, s = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int base = 0; base < n; base += 8) {
        const int cnt = min(8, n - base);
        float l[8];
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u < cnt) {
                const long long i = (long long)(base + u) * stride;
                l[u] = pl[i];
                v[u] = *(const float2*)(po + i * kHeadDim + 2 * lane);
            } else {
                l[u] = -INFINITY;
                v[u] = make_float2(0.0f, 0.0f);
            }
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < 8; ++u) mx = fmaxf(mx, l[u]);
        // every partial so far empty (lse = -inf: a causal row that saw no
        // token): subtract 0 instead of -inf so that the weights come out 0,
        // not NaN
        const float ms = mx == -INFINITY ? 0.0f : mx;
        const float a = __builtin_amdgcn_exp2f(m - ms);    // 0 on the first group (m = -inf)
        s *= a;
        o0 *= a;
        o1 *= a;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w = __builtin_amdgcn_exp2f(l[u] - ms);
            s += w;
            o0 += w * v[u].x;
            o1 += w * v[u].y;
        }
        m = mx;
    }
    const float inv = s > 0.0f ? 1.0f / s : 0.0f;      // a row that saw no token: o = 0
    *(float2*)(out + 2 * lane) = make_float2(o0 * inv, o1 * inv);
    if (lse && lane == 0) *lse = (m + __log2f(s)) * kLn2;
}

// Inclusive prefix over the lanes of each row of 16 (Hillis-Steele with DPP
// row shifts; a lane whose source lies before its row takes `id`).
template <class Op>
__device__ __forceinline__ int row_incl_scan(int v, const int id, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xF, 0xF, false));   // row_shr:1
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xF, 0xF, false));   // row_shr:2
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xF, 0xF, false));   // row_shr:4
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xF, 0xF, false));   // row_shr:8
    return v;
}

// Inclusive sum over the 64 lanes of a wave, in registers: row scans, then
// each row adds the totals of the rows before it (lanes 15, 31, 47).
__device__ __forceinline__ int wave_incl_sum(const int v, const int lane) {
    const int s = row_incl_scan(v, 0, [](int a, int b) { return a + b; });
    const int t0 = __builtin_amdgcn_readlane(s, 15);
    const int t1 = __builtin_amdgcn_readlane(s, 31);
    const int t2 = __builtin_amdgcn_readlane(s, 47);
    const int row = lane >> 4;
    return s + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Minimum / maximum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_min(const int v) {
    const int s = row_incl_scan(v, 0x7FFFFFFF, [](int a, int b) { return min(a, b); });
    return min(min(__builtin_amdgcn_readlane(s, 15), __builtin_amdgcn_readlane(s, 31)),
               min(__builtin_amdgcn_readlane(s, 47), __builtin_amdgcn_readlane(s, 63)));
}
__device__ __forceinline__ int wave_max(const int v) {
    const int s = row_incl_scan(v, (int)0x80000000, [](int a, int b) { return max(a, b); });
    return max(max(__builtin_amdgcn_readlane(s, 15), __builtin_amdgcn_readlane(s, 31)),
               max(__builtin_amdgcn_readlane(s, 47), __builtin_amdgcn_readlane(s, 63)));
}

// Calls seg(b, h, page0, page1, slot, n_segments, lane) for every segment of
// this wave's ranges (split_plan.h).  Must be called by every thread of a
// workgroup of kSplitThreads threads (it synchronises twice); the dynamic LDS
// holds num_seqs + 1 ints.
//
// Balancing.  A segment costs its pages plus a fixed start-up (loading q,
// filling the load pipeline, writing its result), which is worth about
// kSegmentCost pages.  In a batch of unequal lengths each item is therefore
// weighted as pages + kSegmentCost and the weight space, not the page space,
// is cut into equal ranges, so that a wave whose range holds many short items
// gets fewer pages.  The trailing kSegmentCost units of an item hold no pages
// (a range that covers only those is skipped); 8 pages measured best on a
// lognormal-length batch.  When every sequence has the same length the weight
// is 0 and ranges stay aligned with items.  Layout of the shared header: [0] =
// range length (weight units), [1] = the weight.
//
// Order.  Cutting every head's space the same way puts the ranges of all heads
// at one offset (the same pages of the same sequences) on consecutive
// workgroups' waves R apart; with R a multiple of 32 they run on one XCD at
// the same time.  The K/V records of one page's heads are adjacent in the
// pool, so they are read together: the 64-byte sectors two records share are
// fetched once into that XCD's L2, and randomly placed pages still give
// DRAM runs of a whole page's heads.  (A single cut over (sequence, head)
// items spreads a sequence's heads over all XCDs and over time; on a shuffled
// pool of ragged sequences that was 6% slower.)
template <int PS, typename Seg>
__device__ __forceinline__ void for_each_segment(const SplitParams& p, Seg&& seg) {
    extern __shared__ int s_pfx[];   // [num_seqs + 1]
    __shared__ int s_wred[4][kSplitThreads / 64];   // per wave: page sum, items with pages, min, max
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int B = p.num_seqs;

    // One read of the thread's context lengths gives its pages, their sum,
    // the count of items that hold pages and the extremes (is the batch
    // uniform?).  An item weighs pages + K when it holds pages, so the
    // exclusive prefix of the weights is P + K N, with P and N the exclusive
    // prefixes of the pages and of the items with pages: both are scanned
    // before K is known, and one barrier serves the scans and the extremes.
    const int per = (B + kSplitThreads - 1) / kSplitThreads;
    const int beg = min(tid * per, B);
    const int end = min(beg + per, B);
    int psum = 0, nz = 0, pmin = 0x7FFFFFFF, pmax = 0, pg0 = 0;
    for (int i = beg; i < end; ++i) {
        const int pg = pages_of(p.context_lens[i], p.max_ctx, PS);
        if (i == beg) pg0 = pg;
        psum += pg;
        nz += pg > 0 ? 1 : 0;
        pmin = min(pmin, pg);
        pmax = max(pmax, pg);
    }
    const int ps_incl = wave_incl_sum(psum, lane);
    const int nz_incl = wave_incl_sum(nz, lane);
    pmin = wave_min(pmin);
    pmax = wave_max(pmax);
    if (lane == 63) {
        s_wred[0][wid] = ps_incl;
        s_wred[1][wid] = nz_incl;
        s_wred[2][wid] = pmin;
        s_wred[3][wid] = pmax;
    }
    __syncthreads();
    int P = ps_incl - psum, N = nz_incl - nz, Ptot = 0, Ntot = 0;
    for (int w = 0; w < kSplitThreads / 64; ++w) {
        const int sp = s_wred[0][w], sn = s_wred[1][w];
        if (w < wid) {
            P += sp;
            N += sn;
        }
        Ptot += sp;
        Ntot += sn;
        pmin = min(pmin, s_wred[2][w]);
        pmax = max(pmax, s_wred[3][w]);
    }
    const int K = segment_cost(pmin, pmax);
    int run = P + K * N;
    for (int i = beg; i < end; ++i) {
        const int pg = (i == beg) ? pg0 : pages_of(p.context_lens[i], p.max_ctx, PS);
        s_pfx[i] = run;
        run += item_weight(pg, K);
    }
    if (tid == 0) s_pfx[B] = Ptot + K * Ntot;
    __syncthreads();

    const long long S = s_pfx[B];                     // weight of one head's items
    const long long chunk = plan_chunk(S, p.total_waves, p.n_kv, p.min_chunk, p.forced_chunk);
    if (blockIdx.x == 0) {
        if (tid == 0) {
            p.ws_header[0] = (int)chunk;
            p.ws_header[1] = K;
        }
        for (int i = tid; i <= B; i += kSplitThreads) p.ws_pfx[i] = s_pfx[i];
    }

    // Range r of head h is global range h R + r, taken by wave h R + r.
    const long long R = (S + chunk - 1) / chunk;       // ranges per head
    const long long waves = (long long)gridDim.x * (kSplitThreads / 64);
    auto pfx = [&](int i) { return s_pfx[i]; };
    auto uni = [](int v) { return uniform(v); };
    for (long long k = (long long)blockIdx.x * (kSplitThreads / 64) + wid; k < R * p.n_kv; k += waves) {
        const int h = uniform((int)(k / R));
        walk_range(k - (long long)h * R, chunk, S, B, K, pfx, uni,
                   [&](int b, int page0, int page1, int slot, int n_seg) {
                       seg(b, h, page0, page1, slot, n_seg, lane);
                   });
    }
}

}  // namespace kvq
