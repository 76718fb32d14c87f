// append.hip -- quantize-on-append for the FP8 / INT8 paged KV cache (gfx950).
//
// Quantization happens once, when a token's K/V row is stored, from the
// full-precision row, and the per-token scales are kept in BF16 next to the
// codes ("KV 캐시 양자화(KV cache quantization): FP8/INT8 K 및 V가 실제로 제공하는
// 이점과 한계점", molayo1419.me, section "KV 캐시 양자화란 실제로 무엇인가";
// "KV Cache 압축", ryotta.opik.net, sections 5.1 and 6.3).  Formats: FP8 E4M3
// and INT8 per-token asymmetric (scale, zero_point), plus static per-tensor /
// per-head scales (molayo1419.me, formats table notes).
//
// One (token, KV head, K|V) row of 128 bf16 per 8-lane group: each lane loads
// 32 bytes, the row's amax or min/max is combined across the 8 lanes, and each
// lane writes one coalesced 16-byte packed code vector into the page record;
// lane 0 writes the BF16 scale (and zero-point).  The division x / s is one
// correctly rounded IEEE float32 division so that the codes are bit-exact.
#include "kvq_device.h"
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {


template <int DT, bool STATIC, int PS>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = gid >> 3;                 // ((token * n_kv) + head) * 2 + kv
    const int li = threadIdx.x & 7;                 // channels [16 li, 16 li + 16)
    const long long nrows = (long long)p.num_tokens * p.n_kv * 2;
    bool active = row < nrows;
    const int kv = (int)(row & 1);
    const long long th = row >> 1;
    const int tok = (int)(th / p.n_kv);
    const int h = (int)(th - (long long)tok * p.n_kv);
    // the slot and the row are loaded together (the row's address does not
    // depend on the slot)
    long long slot = -1;
    u32x4_t w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (active) {
        slot = p.slot_mapping[tok];
        const uint16_t* src = (kv ? p.v : p.k) + ((size_t)tok * p.n_kv + h) * kHeadDim + 16 * li;
        w0 = *(const u32x4_t*)src;
        w1 = *(const u32x4_t*)(src + 8);
    }
    active = active && slot >= 0 && slot < p.num_slots;
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16lo(w0[i]);
        x[2 * i + 1] = bf16hi(w0[i]);
        x[8 + 2 * i] = bf16lo(w1[i]);
        x[8 + 2 * i + 1] = bf16hi(w1[i]);
    }

    uint32_t code[4];
    uint32_t scale_bits = 0, zero_bits = 0;
    if constexpr (is_fp8_format(DT)) {
        // the per-(token, head) scale maps the row's largest magnitude onto
        // the format's largest finite value
        constexpr float kMaxCode = (DT == kE5M2) ? 57344.0f : 448.0f;
        float sf;
        if constexpr (STATIC) {
            const int idx = kv * p.static_kv_stride + h * p.static_head_stride;
            scale_bits = active ? p.static_scales[idx] : 0u;
            sf = bf16lo(scale_bits);
        } else {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
            amax = group8_extreme<true>(amax);
            scale_bits = bf16_up_bits(amax / kMaxCode);
            sf = bf16lo(scale_bits);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (sf != 0.0f) {
                if constexpr (DT == kE5M2)
                    code[i] = e5m2_encode4(x[4 * i] / sf, x[4 * i + 1] / sf, x[4 * i + 2] / sf,
                                           x[4 * i + 3] / sf);
                else
                    code[i] = e4m3_encode4(x[4 * i] / sf, x[4 * i + 1] / sf, x[4 * i + 2] / sf,
                                           x[4 * i + 3] / sf);
            } else {
                code[i] = 0u;
            }
        }
    } else {
        float lo = x[0], hi = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            lo = fminf(lo, x[i]);
            hi = fmaxf(hi, x[i]);
        }
        lo = group8_extreme<false>(lo);
        hi = group8_extreme<true>(hi);
        zero_bits = bf16_down_bits(lo);
        const float zf = bf16lo(zero_bits);
        const float range = hi - zf;
        scale_bits = bf16_up_bits(range / 255.0f);
        const float sf = bf16lo(scale_bits);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t wv = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t c = 0u;
                if (sf != 0.0f) {
                    float t = rintf((x[4 * i + j] - zf) / sf);
                    t = fminf(fmaxf(t, 0.0f), 255.0f);
                    c = (uint32_t)t;
                }
                wv |= c << (8 * j);
            }
            code[i] = wv;
        }
    }

    if (active) {
        const long long page = slot / PS;
        const int off = (int)(slot - page * PS);
        uint8_t* rec = (kv ? p.v_pages : p.k_pages) +
                       ((size_t)page * p.n_kv + h) * (size_t)(kv ? p.rec_v : p.rec_k);
        u32x4_t cv = {code[0], code[1], code[2], code[3]};
        *(u32x4_t*)(rec + off * kHeadDim + 16 * li) = cv;
        if constexpr (!STATIC) {
            if (li == 0) {
                *(uint16_t*)(rec + PS * kHeadDim + 2 * off) = (uint16_t)scale_bits;
                if constexpr (DT == kINT8)
                    *(uint16_t*)(rec + PS * kHeadDim + 2 * PS + 2 * off) = (uint16_t)zero_bits;
            }
        }
    }
}

template <int DT, bool STATIC, int PS>
static hipError_t launch_append_t(const AppendParams& p, hipStream_t stream) {
    const long long threads = (long long)p.num_tokens * p.n_kv * 2 * 8;
    const long long grid = (threads + 255) / 256;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((append_kernel<DT, STATIC, PS>), dim3((unsigned)grid), dim3(256), 0, stream,
                       p);
    return hipGetLastError();
}

hipError_t launch_append(int dtype, bool static_scale, int page_size, const AppendParams& p,
                         hipStream_t stream) {
    if (dtype == kFP8) {
        if (static_scale)
            return page_size == 16 ? launch_append_t<kFP8, true, 16>(p, stream)
                                   : launch_append_t<kFP8, true, 32>(p, stream);
        return page_size == 16 ? launch_append_t<kFP8, false, 16>(p, stream)
                               : launch_append_t<kFP8, false, 32>(p, stream);
    }
    if (dtype == kE5M2) {
        if (static_scale)
            return page_size == 16 ? launch_append_t<kE5M2, true, 16>(p, stream)
                                   : launch_append_t<kE5M2, true, 32>(p, stream);
        return page_size == 16 ? launch_append_t<kE5M2, false, 16>(p, stream)
                               : launch_append_t<kE5M2, false, 32>(p, stream);
    }
    return page_size == 16 ? launch_append_t<kINT8, false, 16>(p, stream)
                           : launch_append_t<kINT8, false, 32>(p, stream);
}

}  // namespace kvq
