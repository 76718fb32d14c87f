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
    __shared__ int s_wsum[kSplitThreads / 64];
    __shared__ int s_wmin[kSplitThreads / 64], s_wmax[kSplitThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int B = p.num_seqs;

    // pages per sequence, their extremes (is the batch uniform?)
    const int per = (B + kSplitThreads - 1) / kSplitThreads;
    const int beg = min(tid * per, B);
    const int end = min(beg + per, B);
    int pmin = 0x7FFFFFFF, pmax = 0;
    for (int i = beg; i < end; ++i) {
        const int pg = pages_of(p.context_lens[i], p.max_ctx, PS);
        pmin = min(pmin, pg);
        pmax = max(pmax, pg);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        pmin = min(pmin, __shfl_xor(pmin, o));
        pmax = max(pmax, __shfl_xor(pmax, o));
    }
    if (lane == 0) {
        s_wmin[wid] = pmin;
        s_wmax[wid] = pmax;
    }
    __syncthreads();
    for (int w = 0; w < kSplitThreads / 64; ++w) {
        pmin = min(pmin, s_wmin[w]);
        pmax = max(pmax, s_wmax[w]);
    }
    const int K = segment_cost(pmin, pmax);
    auto weight = [&](int i) { return item_weight(pages_of(p.context_lens[i], p.max_ctx, PS), K); };

    // exclusive prefix sum of the per-sequence item weights
    int local = 0;
    for (int i = beg; i < end; ++i) local += weight(i);
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_wsum[wid] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wid; ++w) run += s_wsum[w];
    for (int i = beg; i < end; ++i) {
        s_pfx[i] = run;
        run += weight(i);
    }
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < kSplitThreads / 64; ++w) tot += s_wsum[w];
        s_pfx[B] = tot;
    }
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
