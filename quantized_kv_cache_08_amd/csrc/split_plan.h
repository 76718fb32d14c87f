// split_plan.h -- the flash-decoding work plan, as host-and-device code.
//
// Each (sequence, KV head) is an "item" of pages (32-token chunks for the KIVI
// window path, which counts its fp16 tail as trailing chunks).  For every KV
// head the items of all sequences are laid end to end in a weight space (an
// item weighs its pages plus a fixed start-up cost when the batch is ragged),
// and that space is cut into equal ranges of `chunk` weight units, the same
// cut for every head.  A range is walked item by item; each (item, range)
// overlap that holds pages is a segment.  A segment that covers a whole item
// writes the final result; the others write a partial result into slot
// (range index + sequence index) of their KV head, which is unique: the
// segments of item b sit in consecutive ranges starting at the range that
// holds the item's first weight unit, and every earlier item ends in a range
// no later than that one.  So a head needs at most (ranges + sequences)
// partial slots, whatever the lengths.
//
// The split kernels run this plan on the device (the prefix sums in LDS); the
// test library runs the same functions on the host to check what a plan does
// with a batch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

__host__ __device__ __forceinline__ long long plan_min(long long a, long long b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ long long plan_max(long long a, long long b) { return a > b ? a : b; }

// Pages of context a sequence of `len` tokens occupies (len clamped to max_ctx).
__host__ __device__ __forceinline__ int pages_of(int len, int max_ctx, int ps) {
    len = len < 0 ? 0 : (len > max_ctx ? max_ctx : len);
    return (len + ps - 1) / ps;
}

// Start-up weight of a segment: 0 when every item has the same page count
// (ranges then stay aligned with items), kSegmentCost otherwise.
__host__ __device__ __forceinline__ int segment_cost(int pmin, int pmax) { return pmin == pmax ? 0 : kSegmentCost; }

__host__ __device__ __forceinline__ int item_weight(int pages, int cost) { return pages > 0 ? pages + cost : 0; }

// Range length in weight units for a head weight space of S units.
// forced > 0: that length.  Otherwise one range per resident wave (at most
// kMaxRanges over all heads), and no range shorter than min_chunk.
__host__ __device__ __forceinline__ long long plan_chunk(long long S, int total_waves, int n_kv, int min_chunk,
                                                         int forced) {
    if (forced > 0) return forced;
    const long long waves = plan_min(total_waves, kMaxRanges);
    const long long per_head = plan_max(1, waves / n_kv);
    return plan_max(plan_max((S + per_head - 1) / per_head, min_chunk), 1);
}

// Smallest automatic range for contexts of up to max_pages pages: long enough
// that an item is cut into at most kMaxSegments segments, so that the merge
// of one row stays short.
__host__ __device__ __forceinline__ int plan_min_chunk(int max_pages) {
    int m = kMinChunkPages;
    if (max_pages > kMaxSegments) {
        const int bound = (max_pages + kMaxSegments - 2) / (kMaxSegments - 1);
        m = m > bound ? m : bound;
    }
    return m;
}

// Walks range r of one head: calls f(b, page0, page1, slot, n_seg) for each
// segment, in order.  pfx(i) is the exclusive prefix of item weights (pfx(B)
// = S); uni() makes a value wave-uniform on the device (identity on the host).
template <class Pfx, class Uni, class F>
__host__ __device__ __forceinline__ void walk_range(long long r, long long chunk, long long S, int B, int cost,
                                                    const Pfx& pfx, const Uni& uni, F&& f) {
    long long x = r * chunk;                          // offset inside the head's weight space
    const long long xend = plan_min(x + chunk, S);
    while (x < xend) {
        int lo = 0, hi = B - 1;                       // last item starting at or before x
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((long long)pfx(mid) <= x) lo = mid;
            else hi = mid - 1;
        }
        const int b = uni(lo);
        const int cb = uni(pfx(b + 1) - pfx(b));      // item weight (> 0 here)
        const int pb = cb - cost;                     // item pages
        const long long item_start = pfx(b);
        const long long item_pend = item_start + pb;  // end of the page part
        const long long item_end = item_start + cb;
        if (x < item_pend) {
            const long long seg_end = plan_min(xend, item_pend);
            const int page0 = uni((int)(x - item_start));
            const int page1 = uni((int)(seg_end - item_start));
            const int n_seg = uni((int)((item_pend - 1) / chunk - item_start / chunk + 1));
            const int slot = uni((int)r + b);
            f(b, page0, page1, slot, n_seg);
            x = (seg_end < item_pend) ? seg_end : plan_min(xend, item_end);
        } else {
            x = plan_min(xend, item_end);
        }
    }
}

// Partial-result slots per head that a plan can use: ranges per head plus
// sequences.  Automatic plans have at most max(1, kMaxRanges / n_kv) ranges
// per head (fewer when the whole context is shorter); forced range lengths
// give ceil(S / forced) ranges with S <= B (max_pages + kSegmentCost).
__host__ __device__ __forceinline__ long long plan_slots(int num_seqs, int n_kv, int max_pages, int forced) {
    const long long S_max = (long long)num_seqs * (plan_max(1, max_pages) + kSegmentCost);
    long long ranges;
    if (forced > 0) {
        ranges = (S_max + forced - 1) / forced;
    } else {
        const long long min_chunk = plan_min_chunk(max_pages);
        ranges = plan_min(plan_max(1, kMaxRanges / n_kv), (S_max + min_chunk - 1) / min_chunk);
    }
    return plan_max(1, ranges) + num_seqs;
}

}  // namespace kvq
