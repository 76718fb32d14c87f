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

namespace kvq {

// Merge of the partial results of NH (sequence, query head) rows:
//   L = max_i lse_i,  w_i = 2^(lse_i - L),  out = sum_i w_i o_i / sum_i w_i,
//   lse = (L + log2 sum_i w_i) * ln 2,
// computed online over groups of 8 partial rows.  Called by all 64 lanes of a
// wave; each lane merges channels 2 lane, 2 lane + 1.  Row r's partial lse
// values are pl[r * max_parts + i] and its partial rows po[(r * max_parts + i)
// * 128 + ..], i < n.  All loads of a group (8 lse values and 8 partial rows
// per merged row, every lane reading the same lse words) are issued before
// any is used, so that a merge of up to 8 partials costs one memory round
// trip.
template <int NH>
__device__ __forceinline__ void merge_rows(const float* pl, const float* po, int max_parts, int n,
                                           float* out, float* lse, int lane) {
    float m[NH], s[NH], o0[NH], o1[NH];
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        m[r] = -INFINITY;
        s[r] = 0.0f;
        o0[r] = 0.0f;
        o1[r] = 0.0f;
    }
    for (int base = 0; base < n; base += 8) {
        const int cnt = min(8, n - base);
        float l[NH][8];
        float2 v[NH][8];
#pragma unroll
        for (int r = 0; r < NH; ++r)
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u < cnt) {
                    const float* row = po + ((size_t)r * max_parts + base + u) * kHeadDim + 2 * lane;
                    l[r][u] = pl[(size_t)r * max_parts + base + u];
                    v[r][u] = *(const float2*)row;
                } else {
                    l[r][u] = -INFINITY;
                    v[r][u] = make_float2(0.0f, 0.0f);
                }
            }
#pragma unroll
        for (int r = 0; r < NH; ++r) {
            float mx = m[r];
#pragma unroll
            for (int u = 0; u < 8; ++u) mx = fmaxf(mx, l[r][u]);
            // every partial so far empty (lse = -inf: a causal row that saw no
            // token): subtract 0 instead of -inf so that the weights come out
            // 0, not NaN
            const float ms = mx == -INFINITY ? 0.0f : mx;
            const float a = __builtin_amdgcn_exp2f(m[r] - ms);    // 0 on the first group (m = -inf)
            s[r] *= a;
            o0[r] *= a;
            o1[r] *= a;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float w = __builtin_amdgcn_exp2f(l[r][u] - ms);
                s[r] += w;
                o0[r] += w * v[r][u].x;
                o1[r] += w * v[r][u].y;
            }
            m[r] = mx;
        }
    }
#pragma unroll
    for (int r = 0; r < NH; ++r) {
        const float inv = s[r] > 0.0f ? 1.0f / s[r] : 0.0f;      // a row that saw no token: o = 0
        *(float2*)(out + (size_t)r * kHeadDim + 2 * lane) = make_float2(o0[r] * inv, o1[r] * inv);
        if (lse && lane == 0) lse[r] = (m[r] + __log2f(s[r])) * kLn2;
    }
}

// Pages of context a sequence of `len` tokens occupies (len clamped to max_ctx).
__device__ __forceinline__ int pages_of(int len, int max_ctx, int ps) {
    len = len < 0 ? 0 : (len > max_ctx ? max_ctx : len);
    return (len + ps - 1) / ps;
}

// Calls seg(b, h, page0, page1, seg_index, n_segments, lane) for every
// segment of this wave's ranges.  Must be called by every thread of a
// workgroup of kSplitThreads threads (it synchronises once); the dynamic LDS
// holds num_seqs + 1 ints.
//
// Balancing.  A segment costs its pages plus a fixed start-up (loading q,
// filling the load pipeline, writing its result), which is worth about
// kSegmentCost pages.  In a batch of unequal lengths each item is therefore
// weighted as pages + kSegmentCost and the weight space, not the page space,
// is cut into equal ranges, so that a wave whose range holds many short items
// gets fewer pages.  The trailing kSegmentCost units of an item hold no pages
// (a range that covers only those is skipped); 8 pages measured best on a
// lognormal-length batch.  When every sequence has the
// same length the weight is 0 and ranges stay aligned with items.  Layout of
// the shared header: [0] = range length (weight units), [1] = the weight.
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
    const int K = (pmin == pmax) ? 0 : kSegmentCost;
    auto weight = [&](int i) {
        const int pg = pages_of(p.context_lens[i], p.max_ctx, PS);
        return pg > 0 ? pg + K : 0;
    };

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
    // Each head's weight space [h S, (h + 1) S) is cut into R ranges of `chunk`
    // weight units; range r of head h is global range h R + r.  With R a
    // multiple of 32 and 4 waves per workgroup, the ranges of all heads at the
    // same offset run on the same XCD at the same time, so the heads of one
    // page are read together (one L2, nearby DRAM rows).
    long long chunk;
    if (p.forced_chunk > 0) {
        chunk = p.forced_chunk;
    } else {
        const long long per_head = max(1LL, (long long)p.total_waves / p.n_kv);
        chunk = (S + per_head - 1) / per_head;
        if (chunk < p.min_chunk) chunk = p.min_chunk;
    }
    if (blockIdx.x == 0) {
        if (tid == 0) {
            p.ws_header[0] = (int)chunk;
            p.ws_header[1] = K;
        }
        for (int i = tid; i <= B; i += kSplitThreads) p.ws_pfx[i] = s_pfx[i];
    }

    const long long R = (S + chunk - 1) / chunk;       // ranges per head
    const long long waves = (long long)gridDim.x * (kSplitThreads / 64);
    for (long long k = (long long)blockIdx.x * (kSplitThreads / 64) + wid; k < R * p.n_kv; k += waves) {
        const int h = uniform((int)(k / R));
        long long x = (k - (long long)h * R) * chunk;  // offset inside head h's weight space
        const long long xend = min(x + chunk, S);
        while (x < xend) {
            int lo = 0, hi = B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((long long)s_pfx[mid] <= x) lo = mid;
                else hi = mid - 1;
            }
            const int b = uniform(lo);
            const int cb = uniform(s_pfx[b + 1] - s_pfx[b]);   // item weight (> 0 here)
            const int pb = cb - K;                              // item pages
            const long long item_start = s_pfx[b];
            const long long item_pend = item_start + pb;        // end of the page part
            const long long item_end = item_start + cb;
            if (x < item_pend) {
                const long long seg_end = min(xend, item_pend);
                const int page0 = uniform((int)(x - item_start));
                const int page1 = uniform((int)(seg_end - item_start));
                const long long first_seg = item_start / chunk;
                const int n_seg = uniform((int)((item_pend - 1) / chunk - first_seg + 1));
                const int segi = uniform((int)(x / chunk - first_seg));
                seg(b, h, page0, page1, segi, n_seg, lane);
                x = (seg_end < item_pend) ? seg_end : min(xend, item_end);
            } else {
                x = min(xend, item_end);
            }
        }
    }
}

}  // namespace kvq
