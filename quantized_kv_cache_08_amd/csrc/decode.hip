// decode.hip -- paged FP8 / INT8 decode attention with fused dequantization
// (gfx950), flash-decoding split over the context plus a log-sum-exp merge.
//
// What is computed: for each sequence and query head, softmax attention of the
// one decode query over every cached token, reading the quantized K/V pages
// through the block table and dequantizing inside the kernel, with fp32
// accumulation.  A separate dequantization pass would give back the bandwidth
// saving, so dequantization is fused ("KV Cache 압축", ryotta.opik.net,
// sections 5.1 and 6.3); the attention arithmetic stays in high precision and
// only the bytes shrink ("KV 캐시 양자화(KV cache quantization) ...",
// molayo1419.me, section "KV 캐시 양자화란 실제로 무엇인가" and TL;DR); dot
// products accumulate in fp32 ("KV cache FP8로 동시 요청 76배 수용하기",
// storycompiler.tistory.com, section 4); the cache is paged into fixed-size
// blocks mapped by a per-request table ("FP8 KV Cache부터 INT4 Weight-Only까지",
// daewooki.github.io, core concept 2).
//
// Work decomposition.  Each (sequence, KV head) is an "item" of pages; the
// items are laid end to end and the resulting page space is cut into equal
// ranges, one per resident wave (flash-decoding split over context partitions,
// balanced across the whole batch).  A wave walks its range 32 tokens at a
// time; where a range covers a whole item the result goes straight to `out`,
// otherwise a partial (normalised o, log2-sum-exp) goes to the workspace and
// the reduce kernel merges the partials.
//
// Per 32-token chunk and wave (lane l: j = l % 16, g = l / 16):
//  QK  S^T[token][head] = K[token][:] . Q[head][:] with MFMA 16x16x32 bf16.
//      K codes convert exactly to bf16 (E4M3 through the hardware converter,
//      u8 through fp32), q is bf16, so the products are exact; the per-token
//      scale (and INT8 zero-point times sum(q)) is applied to the fp32 result.
//      A operand: lane (token j, g) holds channels [32g, 32g+32) of its row,
//      loaded as two 16-byte vectors; Q (B operand) is permuted to match.
//  softmax  online, exp2 domain, rescaling only when the running maximum
//      grows by more than 2^8 (values stay exact to fp32 rounding).
//  PV  O[head][chan] += P'[head][token] . V[token][chan], P' = p * v_scale
//      split into bf16 hi + lo (two MFMAs) so P' keeps 16 significant bits.
//      The QK result layout is already the PV A layout (lane = head, slots =
//      tokens 4g..4g+3 of each half); V is loaded as 8-byte row pieces
//      (lane (chan-block j, g): channels 8j..8j+7 of tokens 4g..4g+3) and
//      transposed in registers with byte permutes before conversion.
//
// FP8-domain QK (Q8; the cache descriptor's KVQ_ATTN_FP8_QK flag): some
// serving backends compute attention itself in FP8 ("FP8 KV Cache부터 INT4
// Weight-Only까지", daewooki.github.io, core concept 3).  Here the query row is
// quantized at segment start with the K rows' own rule (s_q = bf16 ceil of
// amax / 448, E4M3 codes of q / s_q, nearest-even) and QK runs on the gfx950
// FP8 MFMA 16x16x128 straight from the loaded K codes (E4M3, or E5M2 as BF8),
// one instruction per 16 tokens with no code conversion; the product of two
// FP8 values is exact in fp32.  The score is s_k s_q (codes . codes).  P and
// PV are unchanged (P' in bf16 hi + lo): E4M3 probabilities, 3 mantissa bits,
// would move outputs far past the 2e-3 bar, and their codes would depend on
// this kernel's running maximum, which no plain definition fixes.
//
// FP8 score-V (PV; the descriptor's KVQ_ATTN_FP8_PV flag, FP8 caches): the
// same page of that section names the score-V product in the FP8 domain too.
// The probabilities of a 32-token chunk, P' = 2^(s - m) v_scale with the
// running maximum m kept an integer, are held as E4M3 codes under the chunk's
// smallest power-of-two scale S with max P' <= 448 S (per query row), and PV
// runs on the scaled FP8 MFMA 16x16x128 straight from the V codes (E4M3, or
// E5M2 as BF8), S entering as the E8M0 scale of the row: one instruction per
// 16 channels, no V conversion.  Because m and the chunk's own reference
// differ by an integer, the codes are those of a definition that does not
// depend on m: the weight of token t relative to its 32-token block's integer
// log2 reference, times its V scale, in E4M3 under the block's power-of-two
// scale.  With page size 16 the work is planned in 32-token units so that a
// segment starts on a block boundary.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "splitk.h"

namespace kvq {

constexpr float kRescaleHeadroom = 8.0f;  // log2 units
constexpr int kBufferFlags = 0x00020000;  // raw buffer resource, dword 3 (gfx9 family)

struct ChunkBuf {
    u32x4_t k[2][2];   // [half][part]: K channels 32g..32g+15 / +16..+31 of token j
    u32x2_t v[2][4];   // [half][r]: V channels 8j..8j+7 of token 4g+r
    u32x2_t ks[2];     // bf16 K scales of tokens 4g..4g+3
    u32x2_t vs[2];
    u32x2_t kz[2];     // INT8 zero-points
    u32x2_t vz[2];
};

// FP8 MFMA 16x16x128: A = 32 FP8 bytes of row l % 16 (format A_FMT: 0 E4M3,
// 1 E5M2), B = 32 E4M3 bytes of column l % 16, the same channels in the same
// byte order on both sides; unit block scales (E8M0 127 = 2^0).
template <int A_FMT>
__device__ __forceinline__ f32x4_t mfma_16x16x128_fp8(const u32x4_t (&a)[2], const uint32_t (&b)[8]) {
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    const i32x8_t av = {(int)a[0][0], (int)a[0][1], (int)a[0][2], (int)a[0][3],
                        (int)a[1][0], (int)a[1][1], (int)a[1][2], (int)a[1][3]};
    const i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, A_FMT, 0, 0, 127, 0, 127);
}

// Scaled FP8 MFMA 16x16x128 for PV: A = 8 E4M3 codes per lane (bytes 0-7 of
// the lane's 32; the rest zero), B = 8 codes of the same tokens (format
// B_FMT: 0 E4M3, 1 E5M2), scale_a = E8M0 exponent of the lane's row (every
// lane of a row carries the same one), B unscaled.
template <int B_FMT>
__device__ __forceinline__ f32x4_t mfma_pv_fp8(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, int scale_a,
                                               f32x4_t c) {
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    const i32x8_t av = {(int)a0, (int)a1, 0, 0, 0, 0, 0, 0};
    const i32x8_t bv = {(int)b0, (int)b1, 0, 0, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, B_FMT, 0, scale_a, 0, 127);
}

// Smallest E with a <= 448 2^E for a finite a >= 0 (0 and float32 subnormals
// give at most -127; the E8M0 range is [-127, 127]):  a = 1.f 2^(e - 127) and
// 448 = 1.75 2^8, so E = e - 135, plus one when 1.f > 1.75.
__device__ __forceinline__ int pow2_scale_exp(float a) {
    const uint32_t u = f32_to_bits(a);
    const int e = (int)(u >> 23) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return min(max(e, -127), 127);
}

// 4 x 4 byte transpose: out[c] byte r = in[r] byte c.
__device__ __forceinline__ void transpose4x4_bytes(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                                   uint32_t (&o)[4]) {
    const uint32_t t0 = perm(v1, v0, 0x05010400u);   // v0.b0 v1.b0 v0.b1 v1.b1
    const uint32_t t1 = perm(v1, v0, 0x07030602u);   // v0.b2 v1.b2 v0.b3 v1.b3
    const uint32_t t2 = perm(v3, v2, 0x05010400u);
    const uint32_t t3 = perm(v3, v2, 0x07030602u);
    o[0] = perm(t2, t0, 0x05040100u);
    o[1] = perm(t2, t0, 0x07060302u);
    o[2] = perm(t3, t1, 0x05040100u);
    o[3] = perm(t3, t1, 0x07060302u);
}

template <int DT, bool STATIC, int PS, bool Q8, bool PV>
__device__ __forceinline__ void process_segment(const SplitParams& p, const int b, const int h,
                                                const int page0, const int page1, const int slot,
                                                const int n_seg, const int lane) {
    const int j = lane & 15;
    const int g = lane >> 4;
    const int G = p.group;
    const int QL = p.q_len;
    const int GQ = G * QL;                 // query rows of this KV head (<= 16)
    const int len = min(max(p.context_lens[b], 0), p.max_ctx);
    const int tok_base = page0 * PS;
    const int tok_end = min(len, page1 * PS);
    // Query row j is position qi = j / G of the QL newest ones (query head
    // h G + j % G) and sees the cache causally: tokens t < len - (QL - 1 - qi).
    // With QL = 1 every row sees the whole context.
    const int qi = j / G;
    const int row_end = min(len - (QL - 1 - min(qi, QL - 1)), page1 * PS);
    const int tail_from = min(len - (QL - 1), page1 * PS);   // first token some row cannot see

    // ---- query operand (B of QK): row j, channels 32g + 8kb + [0, 8)
    u32x4_t qb[4];
    float qsum = 0.0f;
    if (j < GQ) {
        const u32x4_t* qp = (const u32x4_t*)(p.q + (((size_t)b * QL + qi) * p.n_q + (size_t)h * G + (j - qi * G)) *
                                                       kHeadDim +
                                                   32 * g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qb[kb] = qp[kb];
    } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qb[kb] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (DT == kINT8) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) qsum += bf16lo(qb[kb][i]) + bf16hi(qb[kb][i]);
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
    }

    // ---- FP8-domain QK: row j quantized like a K row; byte i of the lane's
    // 32 codes is channel 32g + i (qb[kb] holds channels 32g + 8kb + [0, 8))
    uint32_t qc[8];
    float q_scale = 1.0f;
    if constexpr (Q8) {
#pragma clang fp contract(off)
        float amax = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                amax = fmaxf(amax, fmaxf(fabsf(bf16lo(qb[kb][i])), fabsf(bf16hi(qb[kb][i]))));
        amax = max_over_groups(amax);
        q_scale = bf16lo(bf16_up_bits(amax / 448.0f));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                const uint32_t w0 = qb[kb][2 * i2], w1 = qb[kb][2 * i2 + 1];
                qc[2 * kb + i2] = q_scale != 0.0f
                                      ? e4m3_encode4(bf16lo(w0) / q_scale, bf16hi(w0) / q_scale,
                                                     bf16lo(w1) / q_scale, bf16hi(w1) / q_scale)
                                      : 0u;
            }
    }

    // the query scale (1 unless Q8) multiplies the softmax scale
    const float score_scale = p.score_scale * q_scale;
    float k_static = 0.0f, v_static = 0.0f;
    if constexpr (STATIC) {
        k_static = bf16lo(p.static_scales[h * p.static_head_stride]) * score_scale;
        v_static = bf16lo(p.static_scales[p.static_kv_stride + h * p.static_head_stride]);
    }

    f32x4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // finite, so that a row that sees no token of a chunk (causal rows) gets
    // p = exp2(-inf - m_used) = 0 instead of NaN; any finite score exceeds it
    float m_used = -3.402823466e38f;   // -FLT_MAX
    float lsum = 0.0f;
    float pz = 0.0f;

    // the block table is read-only here: reading it through the constant
    // address space makes the (uniform) page-id loads scalar, so waiting for a
    // page id never waits for the K/V vector loads in flight
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(p.block_table) +
        (size_t)b * p.max_pages_per_seq;
    const int n_chunks = (PS == 16) ? (page1 - page0 + 1) / 2 : (page1 - page0);

    // per-lane byte offsets inside a page record
    const int voff_k = j * kHeadDim + 32 * g;       // K row j, channels [32g, 32g+32)
    const int voff_v = 4 * g * kHeadDim + 8 * j;    // V rows 4g.., channels [8j, 8j+8)
    const int voff_s = PS * kHeadDim + 8 * g;       // bf16 metadata of tokens 4g..4g+3

    // Loads of chunk c through buffer resources spanning one page record.  A
    // chunk or half that does not exist (past the segment, or the second half
    // of an odd page count) gets a zero-size resource: its loads are issued
    // (so every pipeline stage issues the same loads) but fetch nothing and
    // return zeros, and its tokens are masked.
    auto load = [&](ChunkBuf& cb, const int c) {
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            const int pidx = (PS == 16) ? page0 + 2 * c + hp : page0 + c;
            const bool live = (c < n_chunks) && (pidx < page1);
            // page ids come from the caller's table: clamp so that a bad entry
            // reads a wrong page instead of leaving the pool
            const int page = min(max(bt[min(pidx, page1 - 1)], 0), p.num_pages - 1);
            const size_t rec_idx = (size_t)page * p.n_kv + h;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(p.k_pages + rec_idx * (size_t)p.rec_k), (short)0, live ? (int)p.rec_k : 0,
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(p.v_pages + rec_idx * (size_t)p.rec_v), (short)0, live ? (int)p.rec_v : 0,
                kBufferFlags);
            const int t0 = (PS == 16) ? 0 : 16 * hp;     // first token row of this half
            cb.k[hp][0] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k + t0 * kHeadDim, 0, 0);
            cb.k[hp][1] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff_k + t0 * kHeadDim + 16, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                cb.v[hp][r] =
                    __builtin_amdgcn_raw_buffer_load_b64(rv, voff_v + (t0 + r) * kHeadDim, 0, 0);
            if constexpr (!STATIC) {
                cb.ks[hp] = __builtin_amdgcn_raw_buffer_load_b64(rk, voff_s + 2 * t0, 0, 0);
                cb.vs[hp] = __builtin_amdgcn_raw_buffer_load_b64(rv, voff_s + 2 * t0, 0, 0);
                if constexpr (DT == kINT8) {
                    cb.kz[hp] = __builtin_amdgcn_raw_buffer_load_b64(rk, voff_s + 2 * t0 + 2 * PS, 0, 0);
                    cb.vz[hp] = __builtin_amdgcn_raw_buffer_load_b64(rv, voff_s + 2 * t0 + 2 * PS, 0, 0);
                }
            }
        }
    };

    // Only the last chunk of a segment can hold rows past the context end; its
    // masking runs in branches that the empty volatile asm statements keep
    // from being flattened into code that every chunk would execute.
    auto compute = [&](ChunkBuf& cb, const int c) {
        const int ctok = tok_base + c * 32;
        const bool tail = ctok + 32 > tail_from;
        if (__builtin_expect(tail, 0)) {
            __asm__ volatile("");
            // rows past the end of the context may hold anything (including
            // E4M3 NaN patterns): clear them before they reach an MFMA
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ctok + 16 * hp + 4 * g + r >= tok_end) cb.v[hp][r] = u32x2_t{0u, 0u};
        }

        // ---- QK
        float sc[2][4];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            f32x4_t d = {0.f, 0.f, 0.f, 0.f};
            if constexpr (Q8) {
                d = mfma_16x16x128_fp8<DT == kE5M2 ? 1 : 0>(cb.k[hp], qc);
            } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const u32x4_t src = cb.k[hp][kb >> 1];
                const uint32_t d0 = src[(kb & 1) * 2];
                const uint32_t d1 = src[(kb & 1) * 2 + 1];
                u32x4_t a;
                if constexpr (is_fp8_format(DT)) {
                    a = u32x4_t{fp8x2_to_bf16x2<DT, false>(d0), fp8x2_to_bf16x2<DT, true>(d0),
                                fp8x2_to_bf16x2<DT, false>(d1), fp8x2_to_bf16x2<DT, true>(d1)};
                } else {
                    a = u32x4_t{hi_halves(u8_to_f32<0>(d0), u8_to_f32<1>(d0)),
                                hi_halves(u8_to_f32<2>(d0), u8_to_f32<3>(d0)),
                                hi_halves(u8_to_f32<0>(d1), u8_to_f32<1>(d1)),
                                hi_halves(u8_to_f32<2>(d1), u8_to_f32<3>(d1))};
                }
                d = mfma_16x16x32_bf16(a, qb[kb], d);
            }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float s;
                if constexpr (STATIC) {
                    s = d[r] * k_static;
                } else {
                    const uint32_t kw = cb.ks[hp][r >> 1];
                    const float ksr = (r & 1) ? bf16hi(kw) : bf16lo(kw);
                    if constexpr (DT == kINT8) {
                        const uint32_t zw = cb.kz[hp][r >> 1];
                        const float kzr = (r & 1) ? bf16hi(zw) : bf16lo(zw);
                        s = (d[r] * ksr + kzr * qsum) * p.score_scale;
                    } else {
                        s = d[r] * (ksr * score_scale);
                    }
                }
                sc[hp][r] = s;
            }
        }
        if (__builtin_expect(tail, 0)) {
            __asm__ volatile("");
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ctok + 16 * hp + 4 * g + r >= row_end) sc[hp][r] = -INFINITY;
        }

        // ---- online softmax (per head j; all four lane groups agree)
        float mx = sc[0][0];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[hp][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__builtin_expect(__any(mx > m_used + kRescaleHeadroom), 0)) {
            // rare: kept as a branch (an empty volatile asm stops the compiler
            // from flattening it into straight-line code run every chunk)
            __asm__ volatile("");
            // PV: an integer maximum, so that every factor below is a power of two
            const float m_new = PV ? ceilf(fmaxf(m_used, mx)) : fmaxf(m_used, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
            lsum *= alpha;
            pz *= alpha;
            m_used = m_new;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t][r] *= ar;
            }
        }
        float pp[2][4], pzr[2][4];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pr = __builtin_amdgcn_exp2f(sc[hp][r] - m_used);
                lsum += pr;
                float vsr, vzr = 0.0f;
                if constexpr (STATIC) {
                    vsr = v_static;
                } else {
                    const uint32_t vw = cb.vs[hp][r >> 1];
                    vsr = (r & 1) ? bf16hi(vw) : bf16lo(vw);
                    if constexpr (DT == kINT8) {
                        const uint32_t zw = cb.vz[hp][r >> 1];
                        vzr = (r & 1) ? bf16hi(zw) : bf16lo(zw);
                    }
                }
                pp[hp][r] = pr * vsr;
                pzr[hp][r] = pr * vzr;
            }
        }
        if (__builtin_expect(tail, 0)) {
            // masked rows have p = 0, but their scale bytes may be anything
            __asm__ volatile("");
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ctok + 16 * hp + 4 * g + r >= row_end) {
                        pp[hp][r] = 0.0f;
                        pzr[hp][r] = 0.0f;
                    }
        }
        if constexpr (DT == kINT8) {
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r) pz += pzr[hp][r];
        }

        if constexpr (PV) {
            // ---- P' as E4M3 codes under the chunk's power-of-two row scale
            float amax = 0.0f;
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r) amax = fmaxf(amax, pp[hp][r]);
            amax = max_over_groups(amax);
            const int E = pow2_scale_exp(amax);
            uint32_t pc[2];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(pp[hp][0], -E),
                                                        __builtin_amdgcn_ldexpf(pp[hp][1], -E), 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(pp[hp][2], -E),
                                                    __builtin_amdgcn_ldexpf(pp[hp][3], -E), w, true);
                pc[hp] = (uint32_t)w;
            }
            // ---- V codes of channel 8j + t for tokens 4g + r (half hp) in byte r
            uint32_t vt[2][2][4];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int w = 0; w < 2; ++w)
                    transpose4x4_bytes(cb.v[hp][0][w], cb.v[hp][1][w], cb.v[hp][2][w], cb.v[hp][3][w], vt[hp][w]);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[t] = mfma_pv_fp8<DT == kE5M2 ? 1 : 0>(pc[0], pc[1], vt[0][t >> 2][t & 3], vt[1][t >> 2][t & 3],
                                                           E + 127, acc[t]);
            return;
        }

        // ---- P' as bf16 hi + lo (A operands of PV)
        u32x4_t ahi, alo;
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) {
                const float a0 = pp[hp][2 * rp], a1 = pp[hp][2 * rp + 1];
                const uint32_t hw = pack_bf16_rne(a0, a1);
                ahi[2 * hp + rp] = hw;
                alo[2 * hp + rp] = pack_bf16_rne(a0 - bf16lo(hw), a1 - bf16hi(hw));
            }
        }

        // ---- V operands per 16-channel tile and PV
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            u32x4_t bv;
            const int w = t >> 2;
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                if constexpr (is_fp8_format(DT)) {
                    const uint32_t bp = (uint32_t)(t & 2);
                    const uint32_t sel = bp | ((4u + bp) << 8) | ((bp + 1u) << 16) | ((5u + bp) << 24);
                    const uint32_t x01 = perm(cb.v[hp][1][w], cb.v[hp][0][w], sel);
                    const uint32_t x23 = perm(cb.v[hp][3][w], cb.v[hp][2][w], sel);
                    if (t & 1) {
                        bv[2 * hp] = fp8x2_to_bf16x2<DT, true>(x01);
                        bv[2 * hp + 1] = fp8x2_to_bf16x2<DT, true>(x23);
                    } else {
                        bv[2 * hp] = fp8x2_to_bf16x2<DT, false>(x01);
                        bv[2 * hp + 1] = fp8x2_to_bf16x2<DT, false>(x23);
                    }
                } else {
                    const int by = t & 3;
                    const uint32_t v0 = cb.v[hp][0][w], v1 = cb.v[hp][1][w];
                    const uint32_t v2 = cb.v[hp][2][w], v3 = cb.v[hp][3][w];
                    bv[2 * hp] = hi_halves((float)((v0 >> (8 * by)) & 0xFFu),
                                           (float)((v1 >> (8 * by)) & 0xFFu));
                    bv[2 * hp + 1] = hi_halves((float)((v2 >> (8 * by)) & 0xFFu),
                                               (float)((v3 >> (8 * by)) & 0xFFu));
                }
            }
            acc[t] = mfma_16x16x32_bf16(ahi, bv, acc[t]);
            acc[t] = mfma_16x16x32_bf16(alo, bv, acc[t]);
        }
    };

    // ---- software pipeline: one chunk of loads in flight while a chunk is
    // computed (two buffers), for FP8 and INT8 alike.  Launched with one wave
    // per SIMD, this measured faster than INT8 with two chunks in flight
    // (three buffers; 70B shape 724 -> 712 us) and than two waves per SIMD:
    // fewer requests in flight per CU serve the memory system better.
    {
        ChunkBuf b0, b1;
        load(b0, 0);
        for (int c = 0;;) {
            load(b1, c + 1);
            compute(b0, c);
            if (++c >= n_chunks) break;
            load(b0, c + 1);
            compute(b1, c);
            if (++c >= n_chunks) break;
        }
    }

    // ---- epilogue
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if constexpr (DT == kINT8) {
        pz += __shfl_xor(pz, 16);
        pz += __shfl_xor(pz, 32);
    }
    // Rows: output row of query row x is (b QL + x / G) n_q + h G + x % G;
    // a partial result goes to row x of partial slot `slot` of head h.  A row
    // that saw no token (lsum = 0: causal rows of a short context) gives
    // o = 0, lse = -inf.
    const size_t prow0 = ((size_t)h * p.slots + slot) * GQ;
    auto out_row = [&](int x) {
        const int xi = x / G;
        return ((size_t)b * QL + xi) * p.n_q + (size_t)h * G + (x - xi * G);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int head = 4 * g + r;
        const float lr = __shfl(lsum, head & 15);
        const float pzr = (DT == kINT8) ? __shfl(pz, head & 15) : 0.0f;
        if (head < GQ) {
            const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
            f32x4_t o0, o1;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                o0[t] = (acc[t][r] + pzr) * inv;
                o1[t] = (acc[t + 4][r] + pzr) * inv;
            }
            float* dst = (n_seg == 1)
                             ? p.out + out_row(head) * kHeadDim + 8 * j
                             : p.part_o + (prow0 + head) * kHeadDim + 8 * j;
            *(f32x4_t*)dst = o0;
            *(f32x4_t*)(dst + 4) = o1;
        }
    }
    if (g == 0 && j < GQ) {
        const float l2 = lsum > 0.0f ? m_used + __log2f(lsum) : -INFINITY;
        if (n_seg == 1) {
            if (p.lse) p.lse[out_row(j)] = l2 * kLn2;
        } else {
            p.part_lse[prow0 + j] = l2;
        }
    }
}

// PV with page size 16: the plan's unit is a 32-token block (two pages), so
// that every segment starts on a block boundary.
template <int DT, bool STATIC, int PS, bool Q8, bool PV>
__global__ __launch_bounds__(256) void split_kernel(SplitParams p) {
    constexpr int PU = (PV && PS == 16) ? 32 : PS;
    for_each_segment<PU>(p, [&](int b, int h, int page0, int page1, int slot, int n_seg, int lane) {
        if constexpr (PU == PS) {
            process_segment<DT, STATIC, PS, Q8, PV>(p, b, h, page0, page1, slot, n_seg, lane);
        } else {
            const int pages = pages_of(p.context_lens[b], p.max_ctx, PS);
            process_segment<DT, STATIC, PS, Q8, PV>(p, b, h, page0 * (PU / PS), min(page1 * (PU / PS), pages), slot,
                                                    n_seg, lane);
        }
    });
}

// Merge of the partial results of each (sequence, query head), one wave per
// row (merge_row).  Item (b, h)'s partials sit in the consecutive slots of
// head h starting at (range holding the item's first weight unit) + b.
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & 63;
    // idx: query row (b, h, x), x < GQ = group q_len (see the split kernel's
    // epilogue); orow: its output row
    const long long idx = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int GQ = p.group * p.q_len;
    const long long per_seq = (long long)p.n_kv * GQ;
    if (idx >= (long long)p.num_seqs * per_seq) return;
    const int b = (int)(idx / per_seq);
    const int hx = (int)(idx - (long long)b * per_seq);
    const int h = hx / GQ;
    const int x = hx - h * GQ;
    const int xi = x / p.group;
    const long long orow = ((long long)b * p.q_len + xi) * ((long long)p.n_kv * p.group) + (long long)h * p.group +
                           (x - xi * p.group);
    const long long chunk = p.ws_header[0];
    const int cb = p.ws_pfx[b + 1] - p.ws_pfx[b];      // item weight: pages + start-up weight
    if (cb == 0) {
        *(float2*)(p.out + orow * kHeadDim + 2 * lane) = make_float2(0.0f, 0.0f);
        if (p.lse && lane == 0) p.lse[orow] = -INFINITY;
        return;
    }
    const int pb = cb - p.ws_header[1];
    const long long item_start = p.ws_pfx[b];          // offset inside head h's weight space
    const int n_seg = (int)((item_start + pb - 1) / chunk - item_start / chunk + 1);
    if (n_seg == 1) return;   // written by the split kernel
    const size_t prow = ((size_t)h * p.slots + (size_t)(item_start / chunk + b)) * GQ + x;
    merge_row(p.part_lse + prow, p.part_o + prow * kHeadDim, GQ, n_seg, p.out + orow * kHeadDim,
              p.lse ? p.lse + orow : nullptr, lane);
}

template <int DT, bool STATIC, int PS, bool Q8>
static const void* split_fn(bool pv) {
    return pv ? (const void*)&split_kernel<DT, STATIC, PS, Q8, true> : (const void*)&split_kernel<DT, STATIC, PS, Q8, false>;
}

template <int DT, bool STATIC, int PS>
static const void* split_fn(bool q8, bool pv) {
    return q8 ? split_fn<DT, STATIC, PS, true>(pv) : split_fn<DT, STATIC, PS, false>(pv);
}

template <int DT>
static const void* pick_fp8(bool static_scale, int page_size, bool q8, bool pv) {
    if (static_scale) return page_size == 16 ? split_fn<DT, true, 16>(q8, pv) : split_fn<DT, true, 32>(q8, pv);
    return page_size == 16 ? split_fn<DT, false, 16>(q8, pv) : split_fn<DT, false, 32>(q8, pv);
}

// q8 (FP8-domain QK) and pv (FP8 score-V) exist for the FP8 formats only; the
// host refuses them for INT8 caches.
static const void* pick_split(int dtype, bool static_scale, int page_size, bool q8, bool pv) {
    if (dtype == kFP8) return pick_fp8<kFP8>(static_scale, page_size, q8, pv);
    if (dtype == kE5M2) return pick_fp8<kE5M2>(static_scale, page_size, q8, pv);
    return page_size == 16 ? (const void*)&split_kernel<kINT8, false, 16, false, false>
                           : (const void*)&split_kernel<kINT8, false, 32, false, false>;
}

hipError_t split_occupancy(int dtype, bool static_scale, int page_size, bool q8, bool pv, size_t lds_bytes,
                           int* blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, pick_split(dtype, static_scale, page_size, q8, pv), kSplitThreads, lds_bytes);
}

hipError_t launch_split(int dtype, bool static_scale, int page_size, bool q8, bool pv, const SplitParams& p,
                        int grid, size_t lds_bytes, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    SplitParams args = p;
    void* kargs[] = {&args};
    return hipLaunchKernel(pick_split(dtype, static_scale, page_size, q8, pv), dim3(grid),
                           dim3(kSplitThreads), kargs, lds_bytes, stream);
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
    const long long rows = (long long)p.num_seqs * p.n_kv * p.group * p.q_len;
    const long long grid = (rows + 3) / 4;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kvq
