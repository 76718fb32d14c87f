// kvq_internal.h -- parameter blocks and launchers between the C-ABI layer
// (kvq_api.cpp) and the gfx950 kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kMaxSegments = 128;  // most pieces one (sequence, KV head) item is cut into (automatic plan)
constexpr int kMaxRanges = 2048;   // most work ranges (over all KV heads) of one automatic plan
constexpr int kMinChunkPages = 4;  // smallest automatic work range per wave
constexpr int kSegmentCost = 8;    // start-up of a segment, in pages, for ragged batches (measured best on the mixed workload)
constexpr int kSplitThreads = 256; // 4 waves per workgroup
constexpr int kSplitBlocksPerCu = 1;  // FP8 / INT8 split kernel workgroups per CU
constexpr int kKiviGroup = 32;     // KIVI path: tokens per K group = page size

struct AppendParams {
    const uint16_t* k;             // bf16 [T][n_kv][128]
    const uint16_t* v;
    const int32_t* slot_mapping;   // [T]
    uint8_t* k_pages;
    uint8_t* v_pages;
    const uint16_t* static_scales; // bf16 [2][n_kv] (head stride 1) or [2] (stride 0)
    long long rec_k, rec_v;        // record bytes
    long long num_slots;           // num_pages * page_size
    int num_tokens, n_kv, static_head_stride, static_kv_stride;
};

struct SplitParams {
    const uint8_t* k_pages;
    const uint8_t* v_pages;
    const uint16_t* q;             // bf16 [B][q_len][Hq][128]
    const int32_t* block_table;    // [B][max_pages_per_seq]
    const int32_t* context_lens;   // [B]
    const uint16_t* static_scales; // see AppendParams
    float* out;                    // fp32 [B][q_len][Hq][128]
    float* lse;                    // fp32 [B][q_len][Hq] or null
    float* part_o;                 // fp32 [n_kv][slots][group q_len][128]
    float* part_lse;               // fp32 [n_kv][slots][group q_len] (log2 domain)
    int32_t* ws_header;            // [0] = range length, [1] = per-item start-up weight
    int32_t* ws_pfx;               // [B + 1] exclusive prefix of pages per sequence
    long long rec_k, rec_v;
    int num_seqs, n_q, n_kv, group, num_pages;
    int max_pages_per_seq, max_ctx, max_pages;
    int slots;                     // partial-result slots per KV head (>= ranges per head + num_seqs)
    int min_chunk, forced_chunk, total_waves;
    int q_len;                     // query positions per sequence (1: decode; >1: causal verification)
    int static_head_stride, static_kv_stride;
    float score_scale;             // softmax_scale * log2(e)
};

struct ReduceParams {
    const float* part_o;
    const float* part_lse;
    const int32_t* ws_header;
    const int32_t* ws_pfx;
    float* out;
    float* lse;
    int num_seqs, n_q, n_kv, group, slots;
    int q_len;
};

struct KiviAppendParams {
    const uint16_t* k;             // bf16 [total][n_kv][128]
    const uint16_t* v;
    const int32_t* offsets;        // [B + 1]
    const int32_t* context_lens;   // [B] before the append
    const int32_t* block_table;
    uint8_t* k_pages;
    uint8_t* v_pages;
    uint16_t* k_window;            // fp16 [max_seqs][n_kv][W][128]
    uint16_t* v_window;
    long long rec_k, rec_v;
    int num_seqs, n_kv, max_pages_per_seq, window, residual, max_new, num_pages;
    int bits;                      // code width: 4 or 2
};

struct KiviSplitParams {
    SplitParams s;
    const uint16_t* k_window;
    const uint16_t* v_window;
    int window, residual;
    int bits;                      // code width: 4 or 2
};

hipError_t launch_append(int dtype, bool static_scale, int page_size, const AppendParams& p,
                         hipStream_t stream);
hipError_t launch_split(int dtype, bool static_scale, int page_size, bool q8, bool pv, const SplitParams& p,
                        int grid, size_t lds_bytes, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream);
hipError_t split_occupancy(int dtype, bool static_scale, int page_size, bool q8, bool pv, size_t lds_bytes,
                           int* blocks_per_cu);
hipError_t launch_kivi_append(const KiviAppendParams& p, hipStream_t stream);
hipError_t launch_kivi_split(const KiviSplitParams& p, int grid, size_t lds_bytes,
                             hipStream_t stream);
hipError_t kivi_split_occupancy(int bits, int rows, size_t lds_bytes, int* blocks_per_cu);

}  // namespace kvq
