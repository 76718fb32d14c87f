// kvq_api.cpp -- the C ABI of libkvq (declared in include/kvq.h): argument
// validation, page-record accounting, workspace layout, work-range planning
// and kernel launches.  No allocation, no host synchronisation.
#include "kvq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "kvq_internal.h"
#include "split_plan.h"

using namespace kvq;

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int cus = 0;
    void* scratch = nullptr;   // this device's copy of `scratch` (device address)
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_mu;

// Workspace of kvq_decode_attention_noalloc: one copy per device, held from
// module load to process exit.  In host code `scratch` names a host-side
// stand-in; only the address hipGetSymbolAddress returns for the current
// device may reach a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and kept; null on a HIP error.
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_dev[dev].scratch) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_dev[dev].scratch = ptr;
    }
    return g_dev[dev].scratch;
}

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_dev[dev].cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        g_dev[dev].cus = n;
    }
    return g_dev[dev].cus;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool valid_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

bool is_kivi(int dtype) { return dtype == KVQ_INT4_KIVI || dtype == KVQ_INT2_KIVI; }
int kivi_bits(int dtype) { return dtype == KVQ_INT2_KIVI ? 2 : 4; }

// Descriptor checks.  kivi: whether the KIVI window layout is accepted (the
// decode entry points) or refused as unsupported (the slot-based append).
kvq_status check_cache(const kvq_cache* c, bool kivi) {
    if (!c) return KVQ_EINVAL;
    if (c->dtype != KVQ_FP8_E4M3 && c->dtype != KVQ_FP8_E5M2 && c->dtype != KVQ_INT8_ASYM &&
        !is_kivi(c->dtype))
        return KVQ_EINVAL;
    if (c->scale_mode < KVQ_SCALE_PER_TENSOR || c->scale_mode > KVQ_SCALE_PER_TOKEN_HEAD)
        return KVQ_EINVAL;
    if (c->num_pages <= 0 || c->num_kv_heads <= 0 || c->page_size <= 0 || c->head_dim <= 0)
        return KVQ_EINVAL;
    if (!c->k_pages || !c->v_pages) return KVQ_EINVAL;
    if (c->head_dim != kHeadDim) return KVQ_EUNSUPPORTED;
    if (is_kivi(c->dtype)) {
        if (!kivi) return KVQ_EUNSUPPORTED;
        if (c->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD || c->page_size != kKiviGroup)
            return KVQ_EUNSUPPORTED;
        if (!c->k_window || !c->v_window || c->max_seqs <= 0 || c->residual < 0 ||
            c->window_tokens < c->residual + kKiviGroup)
            return KVQ_EINVAL;
        return KVQ_OK;
    }
    if (c->dtype == KVQ_INT8_ASYM && c->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD)
        return KVQ_EUNSUPPORTED;
    if (c->page_size != 16 && c->page_size != 32) return KVQ_EUNSUPPORTED;
    if (c->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD && !c->static_scales) return KVQ_EINVAL;
    return KVQ_OK;
}

// Tokens per unit of the split plan: the page, or with the FP8 score-V
// product on 16-token pages a 32-token block of two pages (a segment then
// starts on a block boundary of that product's probability blocks).
int plan_page_size(const kvq_cache* c) {
    return ((c->attn_flags & KVQ_ATTN_FP8_PV) && c->page_size == 16) ? 32 : c->page_size;
}

struct Plan {
    int max_pages = 0;     // ceil(max_context_len / page_size)
    int slots = 1;         // partial slots per KV head
    int min_chunk = 1;
    int forced_chunk = 0;
    size_t off_pfx = 0, off_lse = 0, off_o = 0, total = 0;
};

// Workspace: a 256-byte header (range length, start-up weight), the prefix of
// item weights [B + 1], then per KV head `slots` partial slots of GQ rows:
// lse [n_kv][slots][GQ] (log2 domain) and o [n_kv][slots][GQ][128] fp32.
Plan make_plan(int page_size, int n_kv, int num_seqs, int num_q_heads, int max_ctx, int partition_pages,
               int q_len) {
    Plan pl;
    pl.max_pages = (max_ctx + page_size - 1) / page_size;
    const int mp = std::max(1, pl.max_pages);
    pl.forced_chunk = partition_pages;
    pl.min_chunk = partition_pages > 0 ? partition_pages : plan_min_chunk(mp);
    const long long slots = plan_slots(num_seqs, n_kv, mp, partition_pages);
    pl.slots = (int)std::min<long long>(slots, 0x7FFFFFFF);
    const size_t rows = (size_t)n_kv * (size_t)slots * (size_t)(num_q_heads / n_kv) * (size_t)q_len;
    pl.off_pfx = 256;
    pl.off_lse = pl.off_pfx + align256(((size_t)num_seqs + 1) * sizeof(int32_t));
    pl.off_o = pl.off_lse + align256(rows * sizeof(float));
    pl.total = pl.off_o + align256(rows * kHeadDim * sizeof(float));
    return pl;
}

kvq_status check_decode(const kvq_cache* c, const void* q, int32_t num_seqs, int32_t num_q_heads,
                        const int32_t* block_table, int32_t max_pages_per_seq,
                        const int32_t* context_lens, int32_t max_context_len,
                        int32_t partition_pages, void* workspace, size_t workspace_bytes,
                        float* out, int32_t q_len, Plan* plan) {
    kvq_status st = check_cache(c, true);
    if (st != KVQ_OK) return st;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_pages_per_seq < 0 ||
        partition_pages < 0 || q_len < 1)
        return KVQ_EINVAL;
    if (num_q_heads % c->num_kv_heads != 0) return KVQ_EINVAL;
    if (c->attn_flags & ~(KVQ_ATTN_FP8_QK | KVQ_ATTN_FP8_PV)) return KVQ_EINVAL;
    if (c->attn_flags && c->dtype != KVQ_FP8_E4M3 && c->dtype != KVQ_FP8_E5M2) return KVQ_EUNSUPPORTED;
    if (!valid_group(num_q_heads / c->num_kv_heads)) return KVQ_EUNSUPPORTED;
    // the query rows of one KV head (group x positions) form one 16-wide MFMA tile
    if ((long long)q_len * (num_q_heads / c->num_kv_heads) > 16) return KVQ_EUNSUPPORTED;
    // KIVI verification: the positions a row cannot see must lie in the fp16
    // window, which holds at least `residual` tokens
    if (q_len > 1 && is_kivi(c->dtype) && q_len - 1 > c->residual) return KVQ_EUNSUPPORTED;
    if ((long long)max_context_len > (long long)max_pages_per_seq * c->page_size)
        return KVQ_EINVAL;
    if (num_seqs > 16383) return KVQ_EUNSUPPORTED;   // prefix table lives in LDS
    if (is_kivi(c->dtype) && num_seqs > c->max_seqs) return KVQ_EINVAL;
    if (num_seqs == 0) return KVQ_OK;
    if (!q || !block_table || !context_lens || !out || !workspace) return KVQ_EINVAL;
    *plan = make_plan(plan_page_size(c), c->num_kv_heads, num_seqs, num_q_heads, max_context_len,
                      partition_pages, q_len);
    if (plan->slots == 0x7FFFFFFF) return KVQ_EUNSUPPORTED;   // forced ranges far too short for the batch
    if (workspace_bytes < plan->total) return KVQ_EWORKSPACE;
    return KVQ_OK;
}

kvq_status run_split(const kvq_cache* c, const void* q, int32_t num_seqs, int32_t num_q_heads,
                     const int32_t* block_table, int32_t max_pages_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                     const Plan& pl, void* workspace, float* out, float* lse, int32_t q_len,
                     hipStream_t stream) {
    const bool is_static = c->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD;
    uint8_t* ws = (uint8_t*)workspace;
    SplitParams p{};
    p.k_pages = (const uint8_t*)c->k_pages;
    p.v_pages = (const uint8_t*)c->v_pages;
    p.q = (const uint16_t*)q;
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.static_scales = (const uint16_t*)c->static_scales;
    p.out = out;
    p.lse = lse;
    p.part_o = (float*)(ws + pl.off_o);
    p.part_lse = (float*)(ws + pl.off_lse);
    p.ws_header = (int32_t*)ws;
    p.ws_pfx = (int32_t*)(ws + pl.off_pfx);
    p.rec_k = (long long)kvq_record_bytes(c->dtype, c->scale_mode, c->page_size, c->head_dim, 0);
    p.rec_v = (long long)kvq_record_bytes(c->dtype, c->scale_mode, c->page_size, c->head_dim, 1);
    p.num_seqs = num_seqs;
    p.n_q = num_q_heads;
    p.n_kv = c->num_kv_heads;
    p.group = num_q_heads / c->num_kv_heads;
    p.num_pages = c->num_pages;
    p.max_pages_per_seq = max_pages_per_seq;
    p.max_ctx = max_context_len;
    p.max_pages = pl.max_pages;
    p.slots = pl.slots;
    p.min_chunk = pl.min_chunk;
    p.forced_chunk = pl.forced_chunk;
    p.q_len = q_len;
    p.static_head_stride = c->scale_mode == KVQ_SCALE_PER_HEAD ? 1 : 0;
    p.static_kv_stride = c->scale_mode == KVQ_SCALE_PER_HEAD ? c->num_kv_heads : 1;
    p.score_scale = softmax_scale * 1.4426950408889634f;

    const size_t lds = ((size_t)num_seqs + 1) * sizeof(int32_t);
    const bool kivi = is_kivi(c->dtype);
    int per_cu = 0;
    const bool q8 = (c->attn_flags & KVQ_ATTN_FP8_QK) != 0;
    const bool pv = (c->attn_flags & KVQ_ATTN_FP8_PV) != 0;
    hipError_t e = kivi ? kivi_split_occupancy(kivi_bits(c->dtype), p.group * q_len, lds, &per_cu)
                        : split_occupancy(c->dtype, is_static, c->page_size, q8, pv, lds, &per_cu);
    if (e != hipSuccess) return KVQ_EHIP;
    const int cus = device_cus();
    if (cus <= 0 || per_cu <= 0) return KVQ_EHIP;
    // FP8 / INT8: one workgroup (one wave per SIMD) per CU, although two fit:
    // with two waves per SIMD the memory system holds more requests than it
    // serves best, and the measured kernel time is 2-3% longer.  KIVI keeps
    // the occupancy limit (two per CU): its pages take more arithmetic per byte.
    const int blocks_per_cu = kivi ? per_cu : std::min(per_cu, kSplitBlocksPerCu);
    const int grid = blocks_per_cu * cus;
    p.total_waves = grid * (kSplitThreads / 64);
    if (kivi) {
        KiviSplitParams kp{};
        kp.s = p;
        kp.k_window = (const uint16_t*)c->k_window;
        kp.v_window = (const uint16_t*)c->v_window;
        kp.window = c->window_tokens;
        kp.residual = c->residual;
        kp.bits = kivi_bits(c->dtype);
        e = launch_kivi_split(kp, grid, lds, stream);
    } else {
        e = launch_split(c->dtype, is_static, c->page_size, q8, pv, p, grid, lds, stream);
    }
    return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status run_reduce(const kvq_cache* c, int32_t num_seqs, int32_t num_q_heads, const Plan& pl,
                      void* workspace, float* out, float* lse, int32_t q_len, hipStream_t stream) {
    uint8_t* ws = (uint8_t*)workspace;
    ReduceParams r{};
    r.part_o = (const float*)(ws + pl.off_o);
    r.part_lse = (const float*)(ws + pl.off_lse);
    r.ws_header = (const int32_t*)ws;
    r.ws_pfx = (const int32_t*)(ws + pl.off_pfx);
    r.out = out;
    r.lse = lse;
    r.num_seqs = num_seqs;
    r.n_q = num_q_heads;
    r.n_kv = c->num_kv_heads;
    r.group = num_q_heads / c->num_kv_heads;
    r.slots = pl.slots;
    r.q_len = q_len;
    return launch_reduce(r, stream) == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

// One decode step: split kernel, then reduce kernel (q_len 1).
kvq_status decode_step(const kvq_cache* cache, const void* q, int32_t num_seqs,
                             int32_t num_q_heads, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* context_lens,
                             int32_t max_context_len, float softmax_scale, int32_t partition_pages,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             hipStream_t stream) {
    Plan pl;
    kvq_status st = check_decode(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq,
                                 context_lens, max_context_len, partition_pages, workspace,
                                 workspace_bytes, out, 1, &pl);
    if (st != KVQ_OK || num_seqs == 0) return st;
    st = run_split(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                   max_context_len, softmax_scale, pl, workspace, out, lse, 1, stream);
    if (st != KVQ_OK) return st;
    return run_reduce(cache, num_seqs, num_q_heads, pl, workspace, out, lse, 1, stream);
}

}  // namespace

extern "C" {

size_t kvq_record_bytes(int32_t dtype, int32_t scale_mode, int32_t page_size, int32_t head_dim,
                        int32_t which) {
    if (page_size <= 0 || head_dim <= 0 || (which != 0 && which != 1)) return 0;
    size_t codes, meta;
    if (dtype == KVQ_FP8_E4M3 || dtype == KVQ_FP8_E5M2) {
        if (scale_mode < KVQ_SCALE_PER_TENSOR || scale_mode > KVQ_SCALE_PER_TOKEN_HEAD) return 0;
        codes = (size_t)page_size * head_dim;
        meta = scale_mode == KVQ_SCALE_PER_TOKEN_HEAD ? 2u * page_size : 0u;
    } else if (dtype == KVQ_INT8_ASYM) {
        if (scale_mode != KVQ_SCALE_PER_TOKEN_HEAD) return 0;
        codes = (size_t)page_size * head_dim;
        meta = 4u * page_size;
    } else if (is_kivi(dtype)) {
        if (scale_mode != KVQ_SCALE_PER_TOKEN_HEAD || (head_dim & 3)) return 0;
        codes = (size_t)page_size * head_dim * kivi_bits(dtype) / 8;
        meta = which == 0 ? 4u * (size_t)head_dim : 4u * page_size;
    } else {
        return 0;
    }
    // padded to 16 bytes; a record of a multiple of 1 KiB (static-scale FP8)
    // gets 32 more, so that a page of records is not a power-of-two stride: the
    // heads of one page are read together and pages of equal-length sequences
    // in lockstep, and a 16 KiB page stride put those reads on the same HBM
    // channels (8B shape: 109 us unpadded, 94 us padded)
    size_t r = (codes + meta + 15) & ~size_t(15);
    if (r % 1024 == 0) r += 32;
    return r;
}

kvq_status kvq_append(const kvq_cache* cache, const void* k, const void* v,
                      const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
    kvq_status st = check_cache(cache, false);
    if (st != KVQ_OK) return st;
    if (num_tokens < 0) return KVQ_EINVAL;
    if (num_tokens == 0) return KVQ_OK;
    if (!k || !v || !slot_mapping) return KVQ_EINVAL;
    AppendParams p{};
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.slot_mapping = slot_mapping;
    p.k_pages = (uint8_t*)cache->k_pages;
    p.v_pages = (uint8_t*)cache->v_pages;
    p.static_scales = (const uint16_t*)cache->static_scales;
    p.rec_k = (long long)kvq_record_bytes(cache->dtype, cache->scale_mode, cache->page_size,
                                          cache->head_dim, 0);
    p.rec_v = (long long)kvq_record_bytes(cache->dtype, cache->scale_mode, cache->page_size,
                                          cache->head_dim, 1);
    p.num_slots = (long long)cache->num_pages * cache->page_size;
    p.num_tokens = num_tokens;
    p.n_kv = cache->num_kv_heads;
    p.static_head_stride = cache->scale_mode == KVQ_SCALE_PER_HEAD ? 1 : 0;
    p.static_kv_stride = cache->scale_mode == KVQ_SCALE_PER_HEAD ? cache->num_kv_heads : 1;
    const bool is_static = cache->scale_mode != KVQ_SCALE_PER_TOKEN_HEAD;
    if (launch_append(cache->dtype, is_static, cache->page_size, p, stream) != hipSuccess)
        return KVQ_EHIP;
    return KVQ_OK;
}

kvq_status kvq_kivi_append(const kvq_cache* cache, const void* k, const void* v,
                           const int32_t* token_offsets, const int32_t* context_lens,
                           const int32_t* block_table, int32_t max_pages_per_seq, int32_t num_seqs,
                           int32_t max_new_tokens, hipStream_t stream) {
    if (!cache) return KVQ_EINVAL;
    if (!is_kivi(cache->dtype)) return check_cache(cache, false) == KVQ_OK
                                                  ? KVQ_EUNSUPPORTED : KVQ_EINVAL;
    kvq_status st = check_cache(cache, true);
    if (st != KVQ_OK) return st;
    if (num_seqs < 0 || max_new_tokens < 0 || max_pages_per_seq < 0) return KVQ_EINVAL;
    if (num_seqs > cache->max_seqs) return KVQ_EINVAL;
    if (num_seqs > 65535 || cache->num_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    if (num_seqs == 0 || max_new_tokens == 0) return KVQ_OK;
    if (!k || !v || !token_offsets || !context_lens || !block_table || max_pages_per_seq == 0)
        return KVQ_EINVAL;
    KiviAppendParams p{};
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.offsets = token_offsets;
    p.context_lens = context_lens;
    p.block_table = block_table;
    p.k_pages = (uint8_t*)cache->k_pages;
    p.v_pages = (uint8_t*)cache->v_pages;
    p.k_window = (uint16_t*)cache->k_window;
    p.v_window = (uint16_t*)cache->v_window;
    p.rec_k = (long long)kvq_record_bytes(cache->dtype, cache->scale_mode, cache->page_size,
                                          cache->head_dim, 0);
    p.rec_v = (long long)kvq_record_bytes(cache->dtype, cache->scale_mode, cache->page_size,
                                          cache->head_dim, 1);
    p.num_seqs = num_seqs;
    p.n_kv = cache->num_kv_heads;
    p.max_pages_per_seq = max_pages_per_seq;
    p.window = cache->window_tokens;
    p.residual = cache->residual;
    p.max_new = max_new_tokens;
    p.num_pages = cache->num_pages;
    p.bits = kivi_bits(cache->dtype);
    return launch_kivi_append(p, stream) == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_decode_workspace_bytes(const kvq_cache* cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      int32_t partition_pages, size_t* bytes) {
    if (!bytes) return KVQ_EINVAL;
    *bytes = 0;
    if (!cache) return KVQ_EINVAL;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_pages < 0)
        return KVQ_EINVAL;
    if (cache->page_size <= 0 || cache->num_kv_heads <= 0 || num_q_heads % cache->num_kv_heads)
        return KVQ_EINVAL;
    *bytes = make_plan(plan_page_size(cache), cache->num_kv_heads, num_seqs, num_q_heads, max_context_len,
                       partition_pages, 1)
                 .total;
    return KVQ_OK;
}

kvq_status kvq_decode_split(const kvq_cache* cache, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, float softmax_scale, int32_t partition_pages,
                            void* workspace, size_t workspace_bytes, float* out, float* lse,
                            hipStream_t stream) {
    Plan pl;
    kvq_status st = check_decode(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq,
                                 context_lens, max_context_len, partition_pages, workspace,
                                 workspace_bytes, out, 1, &pl);
    if (st != KVQ_OK || num_seqs == 0) return st;
    return run_split(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                     max_context_len, softmax_scale, pl, workspace, out, lse, 1, stream);
}

kvq_status kvq_decode_reduce(const kvq_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_context_len, int32_t partition_pages, void* workspace,
                             size_t workspace_bytes, float* out, float* lse, hipStream_t stream) {
    if (!cache) return KVQ_EINVAL;
    if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_pages < 0)
        return KVQ_EINVAL;
    if (cache->num_kv_heads <= 0 || cache->page_size <= 0 || num_q_heads % cache->num_kv_heads)
        return KVQ_EINVAL;
    if (num_seqs == 0) return KVQ_OK;
    if (!workspace || !out) return KVQ_EINVAL;
    Plan pl = make_plan(plan_page_size(cache), cache->num_kv_heads, num_seqs, num_q_heads, max_context_len,
                        partition_pages, 1);
    if (workspace_bytes < pl.total) return KVQ_EWORKSPACE;
    return run_reduce(cache, num_seqs, num_q_heads, pl, workspace, out, lse, 1, stream);
}

kvq_status kvq_decode_attention(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float softmax_scale,
                                int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream) {
    if (cache && is_kivi(cache->dtype)) return KVQ_EUNSUPPORTED;   // kvq_kivi_decode_attention
    return decode_step(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                       max_context_len, softmax_scale, partition_pages, workspace, workspace_bytes, out, lse,
                       stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                        int32_t num_q_heads, const int32_t* block_table,
                                        int32_t max_pages_per_seq, const int32_t* context_lens,
                                        int32_t max_context_len, float softmax_scale,
                                        int32_t partition_pages, float* out, float* lse,
                                        hipStream_t stream) {
    if (cache && is_kivi(cache->dtype)) return KVQ_EUNSUPPORTED;
    void* ws = scratch_ptr();
    if (!ws) return KVQ_EHIP;
    // the plan is checked against the array's size: a larger shape returns
    // KVQ_EWORKSPACE before any launch
    return decode_step(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                       max_context_len, softmax_scale, partition_pages, ws, kScratchBytes, out, lse, stream);
}

kvq_status kvq_kivi_decode_attention(const kvq_cache* cache, const void* q, int32_t num_seqs,
                                     int32_t num_q_heads, const int32_t* block_table,
                                     int32_t max_pages_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, float softmax_scale,
                                     int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                     float* out, float* lse, hipStream_t stream) {
    if (!cache) return KVQ_EINVAL;
    if (!is_kivi(cache->dtype)) return check_cache(cache, false) == KVQ_OK ? KVQ_EUNSUPPORTED : KVQ_EINVAL;
    return decode_step(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                       max_context_len, softmax_scale, partition_pages, workspace, workspace_bytes, out, lse,
                       stream);
}

kvq_status kvq_verify_workspace_bytes(const kvq_cache* cache, int32_t num_seqs, int32_t q_len,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      int32_t partition_pages, size_t* bytes) {
    if (!bytes) return KVQ_EINVAL;
    *bytes = 0;
    if (!cache) return KVQ_EINVAL;
    if (num_seqs < 0 || q_len < 1 || num_q_heads <= 0 || max_context_len < 0 || partition_pages < 0)
        return KVQ_EINVAL;
    if (cache->page_size <= 0 || cache->num_kv_heads <= 0 || num_q_heads % cache->num_kv_heads)
        return KVQ_EINVAL;
    *bytes = make_plan(plan_page_size(cache), cache->num_kv_heads, num_seqs, num_q_heads, max_context_len,
                       partition_pages, q_len)
                 .total;
    return KVQ_OK;
}

kvq_status kvq_verify_split(const kvq_cache* cache, const void* q, int32_t num_seqs, int32_t q_len,
                            int32_t num_q_heads, const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                            int32_t partition_pages, void* workspace, size_t workspace_bytes, float* out,
                            float* lse, hipStream_t stream) {
    Plan pl;
    kvq_status st = check_decode(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq,
                                 context_lens, max_context_len, partition_pages, workspace,
                                 workspace_bytes, out, q_len, &pl);
    if (st != KVQ_OK || num_seqs == 0) return st;
    return run_split(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                     max_context_len, softmax_scale, pl, workspace, out, lse, q_len, stream);
}

kvq_status kvq_verify_reduce(const kvq_cache* cache, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                             int32_t max_context_len, int32_t partition_pages, void* workspace,
                             size_t workspace_bytes, float* out, float* lse, hipStream_t stream) {
    if (!cache) return KVQ_EINVAL;
    if (num_seqs < 0 || q_len < 1 || num_q_heads <= 0 || max_context_len < 0 || partition_pages < 0)
        return KVQ_EINVAL;
    if (cache->num_kv_heads <= 0 || cache->page_size <= 0 || num_q_heads % cache->num_kv_heads)
        return KVQ_EINVAL;
    if ((long long)q_len * (num_q_heads / cache->num_kv_heads) > 16) return KVQ_EUNSUPPORTED;
    if (num_seqs == 0) return KVQ_OK;
    if (!workspace || !out) return KVQ_EINVAL;
    Plan pl = make_plan(plan_page_size(cache), cache->num_kv_heads, num_seqs, num_q_heads, max_context_len,
                        partition_pages, q_len);
    if (workspace_bytes < pl.total) return KVQ_EWORKSPACE;
    return run_reduce(cache, num_seqs, num_q_heads, pl, workspace, out, lse, q_len, stream);
}

kvq_status kvq_verify_attention(const kvq_cache* cache, const void* q, int32_t num_seqs, int32_t q_len,
                                int32_t num_q_heads, const int32_t* block_table,
                                int32_t max_pages_per_seq, const int32_t* context_lens,
                                int32_t max_context_len, float softmax_scale,
                                int32_t partition_pages, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, hipStream_t stream) {
    Plan pl;
    kvq_status st = check_decode(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq,
                                 context_lens, max_context_len, partition_pages, workspace,
                                 workspace_bytes, out, q_len, &pl);
    if (st != KVQ_OK || num_seqs == 0) return st;
    st = run_split(cache, q, num_seqs, num_q_heads, block_table, max_pages_per_seq, context_lens,
                   max_context_len, softmax_scale, pl, workspace, out, lse, q_len, stream);
    if (st != KVQ_OK) return st;
    return run_reduce(cache, num_seqs, num_q_heads, pl, workspace, out, lse, q_len, stream);
}

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid argument";
        case KVQ_EUNSUPPORTED: return "unsupported configuration";
        case KVQ_EWORKSPACE: return "workspace too small";
        case KVQ_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
