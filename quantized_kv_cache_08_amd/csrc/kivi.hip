// kivi.hip -- KIVI-style 4-bit and 2-bit KV cache (gfx950): K quantized per
// channel over groups of 32 tokens, V per token, the most recent tokens kept
// in fp16 ("KV Cache 압축", ryotta.opik.net, section 3.1 KIVI, an asymmetric
// 2-bit method; "KV 캐시 양자화(KV cache quantization) ...", molayo1419.me,
// formats-table notes on mixed-precision 4-bit: K per channel for its channel
// outliers, V per token), with attention over the quantized pages and the
// fp16 window fused into one split-K decode kernel.
//
// Window rule: a sequence of n tokens holds its first
//   n_q = 32 * floor(max(0, n - residual) / 32)
// tokens as 4-bit groups (one 32-token group per page) and tokens [n_q, n)
// as fp16 rows in a ring of `window` >= residual + 32 rows (token t at row
// t % window).  Tokens leave the window whole groups at a time, oldest first.
//
// Quantizer (both K and V; L = 2^bits - 1 = 15 or 3 steps):  z = bf16 floor
//   of the minimum, s = bf16 ceil of (max - z) / L,  code = clamp(rne((x - z)
//   / s), 0, L), x^ = code * s + z, every "/" one IEEE float32 division.  The
//   inputs are the fp16 values (bf16 input rounded to nearest-even fp16).
//
// V records store each token pair's code rows interleaved in 16-bit units:
// word q of pair row m holds channels 4q..4q+3 of token 2m (bits 0-15) and of
// token 2m + 1 (bits 16-31), channel 4q + i in bits 4i..4i+3 of each half.
//
// 2-bit records hold the 4-bit layout at half the rows: every 4-bit field
// carries two codes, bits 0-1 for the first 16 tokens of the page and bits 2-3
// for the last 16 (K row j: tokens j and j + 16; V pair row m: pairs m and
// m + 8).  The decode kernel shifts a field's word by 0 or 2 and masks 2 bits
// where the 4-bit kernel masks 4; the rest of its arithmetic is the same.
//
// Decode of one 32-token page, per wave (lane l: j = l % 16, g = l / 16):
//   score_t = sum_c q_c (n_tc s_c + z_c) = sum_c n_tc (q_c s_c) + sum_c q_c z_c.
//   q'_c = q_c s_c is the product of two bf16 values, at most 16 significant
//   bits, so it splits exactly into bf16 hi + lo; codes enter the MFMA as the
//   bf16 value 128 + n (one byte permute per pair), and the offset
//   128 sum_c q'_c is removed, together with the zero-point term, by
//   bias = sum_c q_c z_c - 128 sum_c q_c s_c from one more small MFMA (rows z
//   and s against q), added where the scores are scaled.
//   PV: O += P'.(128 + n_v) (128 + 8 n_v on odd channels) with P' = p * s_t
//   split into bf16 hi + lo; the offset 128 sum_t P'_t (summed by MFMAs over
//   the same P') and the zero-point term sum_t p_t z_t are removed at the end.
//   fp16 window chunks use fp16 MFMAs on the exact fp16 values.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "splitk.h"

namespace kvq {

constexpr int kKiviBufferFlags = 0x00020000;
constexpr float kKiviHeadroom = 8.0f;      // log2 units

__device__ __forceinline__ int kivi_nq(int n, int resid) {
    const int over = n - resid;
    return over <= 0 ? 0 : (over / kKiviGroup) * kKiviGroup;
}

// ============================================================== append
// Asymmetric quantizer with L steps of one value given the row's (z, s).
template <int L>
__device__ __forceinline__ uint32_t kivi_code(float x, float zf, float sf) {
#pragma clang fp contract(off)
    if (sf == 0.0f) return 0u;
    float t = rintf((x - zf) / sf);
    t = fminf(fmaxf(t, 0.0f), (float)L);
    return (uint32_t)t;
}

// Writes the fp16 window row of new token i of sequence b, KV head h (k or v
// by kv), 8 channels from lane part (16 lanes per row).
__device__ __forceinline__ void kivi_window_row(const KiviAppendParams& p, int b, int h, int i, int kv, int part) {
    const int n0 = max(p.context_lens[b], 0);
    const int m = p.offsets[b + 1] - p.offsets[b];
    const int pos = n0 + i;
    if (i >= m || pos < kivi_nq(n0 + m, p.residual)) return;    // quantized straight from the input
    const size_t src = ((size_t)(p.offsets[b] + i) * p.n_kv + h) * kHeadDim + 8 * part;
    const size_t dst = (((size_t)b * p.n_kv + h) * p.window + pos % p.window) * kHeadDim + 8 * part;
    const u32x4_t w = *(const u32x4_t*)((kv ? p.v : p.k) + src);
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_f16_rne(bf16lo(w[e]), bf16hi(w[e]));
    *(u32x4_t*)((kv ? p.v_window : p.k_window) + dst) = o;
}

// One workgroup quantizes one 32-token group of one (sequence, KV head): K
// per channel (waves 0-1, one thread per channel) and, at the same time, V per
// token (waves 2-3, 16 tokens per wave, two channels per lane).  Token rows
// come from the fp16 window (tokens held before this call) or from the new
// bf16 rows (rounded to fp16).
// ONE_TOKEN (calls that append one token per sequence): workgroup x = 1, which
// has no group to flush then, also writes the new token's window row.  Its
// ring row cannot be one the flush reads: those hold positions p with
// n0 - (residual + 31) <= p < n0, and the ring has window >= residual + 32 rows.
template <int BITS, bool ONE_TOKEN>
__global__ __launch_bounds__(256) void kivi_flush_kernel(KiviAppendParams p) {
#pragma clang fp contract(off)
    constexpr int L = (1 << BITS) - 1;
    constexpr int kCodeBytes = kKiviGroup * kHeadDim * BITS / 8;    // metadata follows the codes
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    if (ONE_TOKEN && blockIdx.x == 1) {
        if (threadIdx.x < 32) kivi_window_row(p, b, h, 0, (int)(threadIdx.x >> 4), (int)(threadIdx.x & 15));
        return;
    }
    const int n0 = max(p.context_lens[b], 0);
    const int m = p.offsets[b + 1] - p.offsets[b];
    if (m <= 0) return;
    const int n1 = n0 + m;
    const int nq0 = kivi_nq(n0, p.residual);
    const int nq1 = kivi_nq(n1, p.residual);
    const int grp = nq0 / kKiviGroup + (int)blockIdx.x;
    if (grp * kKiviGroup >= nq1 || grp >= p.max_pages_per_seq) return;
    const int page = p.block_table[(size_t)b * p.max_pages_per_seq + grp];
    if (page < 0 || page >= p.num_pages) return;
    const int tid = threadIdx.x;
    const size_t wrow0 = ((size_t)b * p.n_kv + h) * p.window;
    const int in0 = p.offsets[b];

    // Token t of the group: window row (t0 + t) mod window if it was held before
    // this call, else new input row.  The source is selected per token (uniform)
    // and the 16-bit word converted after the load, so that all of a thread's
    // loads are in flight together.
    const int base = grp * kKiviGroup;
    const int r0 = base % p.window;
    auto src = [&](const uint16_t* win, const uint16_t* in, int t, int c) -> const uint16_t* {
        const int pos = base + t;
        int r = r0 + t;
        if (r >= p.window) r -= p.window;              // t < 32 <= window
        return pos < n0 ? win + (wrow0 + r) * kHeadDim + c
                        : in + ((size_t)(in0 + max(pos - n0, 0)) * p.n_kv + h) * kHeadDim + c;
    };
    auto value = [&](uint16_t w, int t) -> float {
        return base + t < n0 ? f16_value(w) : (float)(_Float16)bf16lo(w);
    };

    uint8_t* krec = p.k_pages + ((size_t)page * p.n_kv + h) * (size_t)p.rec_k;
    uint8_t* vrec = p.v_pages + ((size_t)page * p.n_kv + h) * (size_t)p.rec_v;
    if (tid < kHeadDim) {
        // ---- K: channel c over the group's 32 tokens
        const int c = tid;
        uint16_t wv[kKiviGroup];
#pragma unroll
        for (int t = 0; t < kKiviGroup; ++t) wv[t] = *src(p.k_window, p.k, t, c);
        float x[kKiviGroup];
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int t = 0; t < kKiviGroup; ++t) {
            x[t] = value(wv[t], t);
            lo = fminf(lo, x[t]);
            hi = fmaxf(hi, x[t]);
        }
        const uint32_t zb = bf16_down_bits(lo);
        const float zf = bf16lo(zb);
        const uint32_t sb = bf16_up_bits((hi - zf) / (float)L);
        const float sf = bf16lo(sb);
        // row r holds token r (4 bits) or tokens r and r + 16 (2 + 2 bits)
        constexpr int kRows = BITS == 4 ? kKiviGroup : kKiviGroup / 2;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            uint32_t code = kivi_code<L>(x[r], zf, sf);
            if constexpr (BITS == 2) code |= kivi_code<L>(x[r + kRows], zf, sf) << 2;
            const uint32_t other = dpp_mov<0xB1>(code);   // quad_perm [1,0,3,2]: lane c ^ 1
            if ((c & 1) == 0) krec[r * (kHeadDim / 2) + (c >> 1)] = (uint8_t)(code | (other << 4));
        }
        *(uint16_t*)(krec + kCodeBytes + 2 * c) = (uint16_t)sb;
        *(uint16_t*)(krec + kCodeBytes + 2 * kHeadDim + 2 * c) = (uint16_t)zb;
    }

    else {
        // ---- V: token t over its 128 channels (one wave per 16 tokens, two
        // channels per lane; all 32 loads of a lane first).  4 bits: wave w
        // takes tokens 16w + i.  2 bits: tokens 8w + i / 2 + 16 (i & 1), so that
        // the two tokens sharing a code byte (t and t + 16) are in one lane.
        const int w = (tid - kHeadDim) >> 6;
        const int l = tid & 63;
        auto tok = [&](int i) { return BITS == 4 ? w * (kKiviGroup / 2) + i : 8 * w + (i >> 1) + 16 * (i & 1); };
        uint32_t wv[kKiviGroup / 2];
#pragma unroll
        for (int i = 0; i < kKiviGroup / 2; ++i) {
            const uint16_t* a = src(p.v_window, p.v, tok(i), 2 * l);
            wv[i] = (uint32_t)a[0] | ((uint32_t)a[1] << 16);
        }
        uint32_t c0[kKiviGroup / 2], c1[kKiviGroup / 2];
#pragma unroll
        for (int i = 0; i < kKiviGroup / 2; ++i) {
            const int t = tok(i);
            const float x0 = value((uint16_t)(wv[i] & 0xFFFFu), t);
            const float x1 = value((uint16_t)(wv[i] >> 16), t);
            const float lo = wave_extreme<false>(fminf(x0, x1));
            const float hi = wave_extreme<true>(fmaxf(x0, x1));
            const uint32_t zb = bf16_down_bits(lo);
            const float zf = bf16lo(zb);
            const uint32_t sb = bf16_up_bits((hi - zf) / (float)L);
            const float sf = bf16lo(sb);
            c0[i] = kivi_code<L>(x0, zf, sf);
            c1[i] = kivi_code<L>(x1, zf, sf);
            if (l == 0) {
                *(uint16_t*)(vrec + kCodeBytes + 2 * t) = (uint16_t)sb;
                *(uint16_t*)(vrec + kCodeBytes + 2 * kKiviGroup + 2 * t) = (uint16_t)zb;
            }
        }
        // token pairs interleaved in 16-bit units: pair row t / 2, channel quad l / 2
#pragma unroll
        for (int i = 0; i < kKiviGroup / 2; i += (BITS == 4 ? 1 : 2)) {
            const int t = tok(i);
            uint32_t b0 = c0[i], b1 = c1[i];
            if constexpr (BITS == 2) {
                b0 |= c0[i + 1] << 2;     // token t + 16
                b1 |= c1[i + 1] << 2;
            }
            vrec[(t >> 1) * kHeadDim + 4 * (l >> 1) + 2 * (t & 1) + (l & 1)] = (uint8_t)(b0 | (b1 << 4));
        }
    }
}

// New tokens that stay in full precision: fp16 rows into the window ring.
// 16 threads per (token, KV head) row, 8 channels each.  Runs after the
// flush kernel, which may still read window rows this kernel overwrites.
__global__ __launch_bounds__(256) void kivi_window_kernel(KiviAppendParams p) {
    const int i = (int)blockIdx.x * 16 + (int)(threadIdx.x >> 4);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) kivi_window_row(p, blockIdx.z, blockIdx.y, i, kv, threadIdx.x & 15);
}

hipError_t launch_kivi_append(const KiviAppendParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0 || p.max_new <= 0) return hipSuccess;
    if (p.bits != 4 && p.bits != 2) return hipErrorInvalidValue;
    const int groups = (p.max_new + kKiviGroup - 1) / kKiviGroup + 1;
    const dim3 grid(groups, p.n_kv, p.num_seqs);
    if (p.max_new == 1) {      // one launch: flush and window row (see kivi_flush_kernel)
        if (p.bits == 4) hipLaunchKernelGGL((kivi_flush_kernel<4, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((kivi_flush_kernel<2, true>), grid, dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    if (p.bits == 4) hipLaunchKernelGGL((kivi_flush_kernel<4, false>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((kivi_flush_kernel<2, false>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kivi_window_kernel, dim3((p.max_new + 15) / 16, p.n_kv, p.num_seqs), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

// ============================================================== decode
// Per-page loads into registers: the 4-bit codes, and the page's scales and
// zero-points as three words per lane (the whole 640-byte metadata block of
// the K and V records), which the wave spreads through its LDS slot when it
// computes the page.  A pipeline stage is 19 VGPRs.
struct KiviBuf {
    u32x4_t kc[2];     // [half]: K codes of token 16 hp + j, channels [32g, 32g+32)
    u32x2_t vc[2][2];  // [half][rp]: V token pair 8 hp + 2g + rp, channels [8j, 8j+8)
    uint32_t km[2];    // K record bytes 2048 + 4 lane and 2304 + 4 lane (scales, zero-points)
    uint32_t vm;       // V record bytes 2048 + 4 lane (scales, zero-points; 0 past the record)
};

// LDS slot of one wave: [0, 256) K scales (128 bf16), [256, 512) K
// zero-points (bf16), [512, 1024) K scales as fp32, [1024, 1152) V scales as
// fp32 (32 tokens), [1152, 1280) V zero-points as fp32, [1280, 1536) unused
// (written with the zeros that lanes 32-63 load past the V record).
constexpr int kKiviMetaBytes = 1536;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;

struct KiviState {
    f32x4_t acc[8];    // O rows (heads 4g + r) x channel 8j + t; odd t carry codes x 8
    f32x4_t pc;        // sum of the P' values the PV products consumed, rows 4g + r
    float m_used, lsum, pz;
};

// Rescale of the running state when a chunk's maximum mx (equal on all lanes
// of a head) exceeds m_used by more than the headroom.
__device__ __forceinline__ void kivi_rescale(KiviState& st, const float mx, const int g) {
    if (__builtin_expect(__any(mx > st.m_used + kKiviHeadroom), 0)) {
        __asm__ volatile("");   // keep the rare rescale a branch, not straight-line code
        const float m_new = fmaxf(st.m_used, mx);
        const float alpha = __builtin_amdgcn_exp2f(st.m_used - m_new);
        st.lsum *= alpha;
        st.pz *= alpha;
        st.m_used = m_new;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * g + r);
            st.pc[r] *= ar;
#pragma unroll
            for (int t = 0; t < 8; ++t) st.acc[t][r] *= ar;
        }
    }
}

// Online-softmax update with the scores of one 32-token chunk (exp2 domain);
// returns p per (half, r) in pp.  All four lane groups hold the same head.
// keep = false: the lane's column duplicates another lane's head; it follows
// the maximum but contributes p = 0.
__device__ __forceinline__ void kivi_softmax(KiviState& st, float (&sc)[2][4], float (&pp)[2][4],
                                             const int g, const bool keep) {
    float mx = sc[0][0];
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[hp][r]);
    kivi_rescale(st, max_over_groups(mx), g);
#pragma unroll
    for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = keep ? __builtin_amdgcn_exp2f(sc[hp][r] - st.m_used) : 0.0f;
            st.lsum += pr;
            pp[hp][r] = pr;
        }
}

// Lane j of each row of 16 takes the word of lane (j + 8) mod 16.
__device__ __forceinline__ uint32_t row_swap8(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);   // row_ror:8
}

// Lanes of the DPP banks in BANKS (four lanes each: 0xC = lanes 8-15 of a row
// of 16, 0x3 = lanes 0-7) take src of lane (j + 8) mod 16; the others keep keep.
template <int BANKS>
__device__ __forceinline__ uint32_t row_swap8_into(uint32_t keep, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)src, 0x128, 0xF, BANKS, false);
}

// (w & mask) | c as one v_and_or_b32: the mask is held in a VGPR and c in an
// SGPR (a VOP3 instruction takes no literal here), both opaque to the
// compiler so that it neither rematerialises them nor splits the expression
// into two literal-operand instructions.  Plain code, not inline assembly: the
// compiler's hazard checks must see these writes of MFMA operands.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t vmask, uint32_t c) {
    return (w & vmask) | c;
}

// The same update when lanes j and j + 8 of a row share head j % 8, each
// holding four of its scores (tokens 4g + r of one 16-token half).
__device__ __forceinline__ void kivi_softmax_half(KiviState& st, const float (&sc)[4], float (&pp)[4],
                                                  const int g) {
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_over_groups(mx);
    mx = fmaxf(mx, bits_to_f32(row_swap8(f32_to_bits(mx))));
    kivi_rescale(st, mx, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pp[r] = __builtin_amdgcn_exp2f(sc[r] - st.m_used);
        st.lsum += pp[r];
    }
}

// V code pairs -> bf16 operand words.  Word w holds a token pair's codes of
// four channels, the pair's first token in bits [0, 16), the second in
// [16, 32), channel 4q + i in bits [4i, 4i + 4) of each half.  Channel
// positions 0 and 2 become bf16 128 + n, positions 1 and 3 bf16 128 + 8n.
// m0 = 0x000F000F, m1 = 0x00780078 (4-bit fields; 0x00030003, 0x00180018 for
// 2-bit codes in the low bits of the fields), held in VGPRs; c = 0x43004300
// (bf16 128 twice) in an SGPR.
template <int POS>
__device__ __forceinline__ uint32_t v_pair(uint32_t w, uint32_t m0, uint32_t m1, uint32_t c) {
    if constexpr (POS == 0) return and_or(w, m0, c);
    if constexpr (POS == 1) return and_or(w >> 1, m1, c);
    if constexpr (POS == 2) return and_or(w >> 8, m0, c);
    return and_or(w >> 9, m1, c);
}

// SHARE (query group <= 8): lanes j and j + 8 hold the same head and each
// forms q' = q s for half of the channel blocks.  The bf16 hi parts of head
// j's q' (and of its P') then take column (row) j of the 16-wide tiles and the
// lo parts column (row) j + 8, so one MFMA forms both products: column j + 8's
// score part is added to column j's, and the accumulator rows 8-15 to rows 0-7
// once, in the epilogue.
// BITS = 2: one load brings a lane's codes of both token halves (hp = 0, 1),
// in bits 0-1 and 2-3 of each 4-bit field; the buffers' [0] entries hold them.
constexpr int kFoldPages = 16;   // pages between folds of the code offset (a power of two)

template <int BITS, bool SHARE>
__device__ __forceinline__ void kivi_segment(const KiviSplitParams& kp, const int b, const int h,
                                             const int page0, const int page1, const int slot,
                                             const int n_seg, const int lane, lds_u8* smeta,
                                             const lds_u8* szero) {
    const SplitParams& p = kp.s;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int G = p.group;
    const int QL = p.q_len;
    const int GQ = G * QL;                       // query rows of this KV head (verification: QL > 1)
    const int hj = SHARE ? (j & 7) : j;          // query row of this lane
    const int len = min(max(p.context_lens[b], 0), p.max_ctx);
    const int nq = kivi_nq(len, kp.residual);
    const int pq = nq / kKiviGroup;
    // Row hj is position qi = hj / G of the QL newest (query head h G + hj % G)
    // and sees tokens t < row_end.  The host requires QL - 1 <= residual, so
    // every row sees all quantized tokens (nq <= len - residual): only fp16
    // window chunks are masked.
    const int qi = hj / G;
    const int row_end = len - (QL - 1 - min(qi, QL - 1));

    // query (B operand): row hj, channels 32g + 8kb + [0, 8)
    u32x4_t qb[4];
    if (hj < GQ) {
        const u32x4_t* qp = (const u32x4_t*)(p.q + (((size_t)b * QL + qi) * p.n_q + (size_t)h * G + (hj - qi * G)) *
                                                       kHeadDim +
                                                   32 * g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qb[kb] = qp[kb];
    } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qb[kb] = u32x4_t{0u, 0u, 0u, 0u};
    }

    // fp32 query values of the channel blocks whose q' this lane forms:
    // blocks kb0 + kk (kb0 = 0, or 2 on lanes 8-15 when sharing)
    constexpr int NKB = SHARE ? 2 : 4;
    const int kb0 = SHARE ? 2 * (j >> 3) : 0;
    float qf[NKB][8];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w = qb[kk][i];
            if constexpr (SHARE) w = (j >= 8) ? qb[kk + 2][i] : w;
            qf[kk][2 * i] = bf16lo(w);
            qf[kk][2 * i + 1] = bf16hi(w);
        }

    KiviState st;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.pc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // finite, so that a row that sees no token of a chunk (causal rows) gets
    // p = exp2(-inf - m_used) = 0 instead of NaN
    st.m_used = -3.402823466e38f;   // -FLT_MAX
    st.lsum = 0.0f;
    st.pz = 0.0f;

    // read-only block table through the constant address space: page-id loads
    // are scalar and never wait for the K/V vector loads in flight
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(p.block_table) + (size_t)b * p.max_pages_per_seq;
    const int qend = min(page1, pq);            // quantized pages of this segment: [page0, qend)
    const int n_q = qend - page0;
    const uint32_t kC = 0x43434343u;           // bf16 high byte of 128 + n
    const u32x4_t kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const uint32_t neg_lo = opaque_sgpr(0x0000BF80u), neg_hi = opaque_sgpr(0xBF800000u);   // bf16 (-1, 0), (0, -1)
    // V code masks, opaque to the compiler so that they stay in two VGPRs
    // instead of being rematerialised before every and_or
    uint32_t vm0 = BITS == 4 ? 0x000F000Fu : 0x00030003u, vm1 = BITS == 4 ? 0x00780078u : 0x00180018u;
    __asm__("" : "+v"(vm0));
    __asm__("" : "+v"(vm1));
    const uint32_t vc128 = opaque_sgpr(0x43004300u);          // bf16 (128, 128)

    const int off_kc = j * (kHeadDim / 2) + 16 * g;
    const int off_vc = (2 * g) * (2 * kHeadDim / 2) + 8 * j;
    constexpr int kPairBytes = 2 * kHeadDim / 2;                   // one V token pair
    constexpr int kMetaOff = kKiviGroup * kHeadDim * BITS / 8;   // metadata after the codes
    constexpr int kHalves = BITS == 4 ? 2 : 1;                    // code loads per page and lane

    auto load = [&](KiviBuf& cb, const int c) {
        const bool live = c < n_q;
        const int pidx = page0 + min(c, max(n_q - 1, 0));
        const int page = min(max(bt[pidx], 0), p.num_pages - 1);
        const size_t rec_idx = (size_t)page * p.n_kv + h;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.k_pages + rec_idx * (size_t)p.rec_k), (short)0, live ? (int)p.rec_k : 0,
            kKiviBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.v_pages + rec_idx * (size_t)p.rec_v), (short)0, live ? (int)p.rec_v : 0,
            kKiviBufferFlags);
#pragma unroll
        for (int hp = 0; hp < kHalves; ++hp)
            cb.kc[hp] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_kc + hp * 16 * (kHeadDim / 2), 0, 0);
#pragma unroll
        for (int hp = 0; hp < kHalves; ++hp)
#pragma unroll
            for (int rp = 0; rp < 2; ++rp)
                cb.vc[hp][rp] = __builtin_amdgcn_raw_buffer_load_b64(
                    rv, off_vc + (8 * hp + rp) * kPairBytes, 0, 0);
        cb.km[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, kMetaOff + 4 * lane, 0, 0);
        cb.km[1] = __builtin_amdgcn_raw_buffer_load_b32(rk, kMetaOff + 256 + 4 * lane, 0, 0);
        cb.vm = __builtin_amdgcn_raw_buffer_load_b32(rv, kMetaOff + 4 * lane, 0, 0);
    };

    // A page is computed in three parts so that the loop can overlap one
    // page's PV products (back) with the next page's QK work (front):
    //   front: metadata to LDS, bias, q' = q s, QK products;
    //   mid:   softmax and P' (state update; holds the rare rescale branch);
    //   back:  offset sums and PV products of a page whose mid has run.
    struct Front {
        f32x4_t dq[2];
        f32x4_t vsf[2], vzf[2];
        float bias_s;
    };
    struct Pend {
        u32x2_t vc[2][2];
        u32x4_t ahi, alo;
    };
    auto front = [&](KiviBuf& cb, Front& F) {
        // spread the page's metadata through the wave's LDS slot (the wave's LDS
        // operations execute in order: the reads below see these writes, and the
        // previous page's reads were issued before them)
        *(lds_u32*)(smeta + 4 * lane) = cb.km[0];
        *(lds_u32*)(smeta + 256 + 4 * lane) = cb.km[1];
        *(lds_u32x2*)(smeta + 512 + 8 * lane) = u32x2_t{cb.km[0] << 16, cb.km[0] & 0xFFFF0000u};
        *(lds_u32x2*)(smeta + 1024 + 8 * lane) = u32x2_t{cb.vm << 16, cb.vm & 0xFFFF0000u};
        const lds_u8* m = smeta;
        u32x4_t kz[4];
        // rows 4i of the bias tile are the zero-points, rows 4i + 1 the scales, so
        // that every lane group finds its column's two sums in d2[0], d2[1]
        const lds_u8* zsrc = ((j & 3) == 0) ? m + 256 + 64 * g : ((j & 3) == 1 ? m + 64 * g : szero);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) kz[kb] = *(const lds_u32x4*)(zsrc + 16 * kb);
        f32x4_t sf[NKB][2];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                sf[kk][x] = *(const lds_f32x4*)(m + 512 + 4 * (32 * g + 8 * (kb0 + kk) + 4 * x));
        // V scales / zero-points of tokens 16 hp + 4g + [0, 4); when sharing, a
        // lane needs only its own half hp = j / 8
#pragma unroll
        for (int hp = 0; hp < (SHARE ? 1 : 2); ++hp) {
            const int hq = SHARE ? (j >> 3) : hp;
            F.vsf[hp] = *(const lds_f32x4*)(m + 1024 + 4 * (16 * hq + 4 * g));
            F.vzf[hp] = *(const lds_f32x4*)(m + 1152 + 4 * (16 * hq + 4 * g));
        }

        // bias = sum_c q_c z_c - 128 sum_c q_c s_c for head j, added to the
        // scaled scores (not used as the accumulators' start, so that the QK
        // products do not wait for it)
        f32x4_t d2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) d2 = mfma_16x16x32_bf16(kz[kb], qb[kb], d2);
        F.bias_s = (d2[0] - 128.0f * d2[1]) * p.score_scale;

        // q' = q s, exact in fp32 (at most 16 significant bits): its bf16
        // rounding and the remainder are both exact bf16 values; slots ordered
        // like the code bytes (channel pairs (0,2), (1,3), (4,6), (5,7) of a block)
        u32x4_t bh[NKB], bl[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
            float a[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) a[c] = qf[kk][c] * sf[kk][c >> 2][c & 3];
            const int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u32x2_t hl = split_bf16(a[ord[2 * e]], a[ord[2 * e + 1]], neg_lo, neg_hi);
                bh[kk][e] = hl[0];
                bl[kk][e] = hl[1];
            }
        }
        u32x4_t BH[4], BL[4];
        if constexpr (SHARE) {
            // lanes j hold blocks 0-1, lanes j + 8 blocks 2-3: column j gets the
            // hi parts of all four, column j + 8 the lo parts
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    BH[kk][e] = row_swap8_into<0xC>(bh[kk][e], bl[kk][e]);
                    BH[2 + kk][e] = row_swap8_into<0x3>(bl[kk][e], bh[kk][e]);
                }
        } else {
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk) {
                BH[kk] = bh[kk];
                BL[kk] = bl[kk];
            }
        }

#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
            f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                uint32_t x, y;
                if constexpr (BITS == 4) {
                    const uint32_t w = cb.kc[hp][kb];
                    x = w & 0x0F0F0F0Fu;
                    y = (w >> 4) & 0x0F0F0F0Fu;
                } else {
                    const uint32_t w = cb.kc[0][kb];
                    x = (w >> (2 * hp)) & 0x03030303u;
                    y = (w >> (4 + 2 * hp)) & 0x03030303u;
                }
                const u32x4_t a = {perm(kC, x, 0x04010400u), perm(kC, y, 0x04010400u),
                                   perm(kC, x, 0x04030402u), perm(kC, y, 0x04030402u)};
                d = mfma_16x16x32_bf16(a, BH[kb], d);
                if constexpr (!SHARE) d = mfma_16x16x32_bf16(a, BL[kb], d);
            }
            F.dq[hp] = d;
        }
    };

    auto mid = [&](const Front& F, const KiviBuf& cb, Pend& pd) {
        const f32x4_t* dq = F.dq;
        const f32x4_t* vsf = F.vsf;
        const f32x4_t* vzf = F.vzf;
        const float bias_s = F.bias_s;
        u32x4_t ahi, alo;
        if constexpr (SHARE) {
            // Lanes j take the first half (tokens 4g + r) of head j's scores and
            // lanes j + 8 the second (tokens 16 + 4g + r): each adds its half's hi
            // part (column j) and lo part (column j + 8), so each lane
            // exponentiates and splits four scores.
            float sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t d0 = f32_to_bits(dq[0][r]), d1 = f32_to_bits(dq[1][r]);
                const float dhi = bits_to_f32(row_swap8_into<0xC>(d0, d1));
                const float dlo = bits_to_f32(row_swap8_into<0x3>(d1, d0));
                sc[r] = __builtin_fmaf(dhi + dlo, p.score_scale, bias_s);
            }
            float pp[4];
            kivi_softmax_half(st, sc, pp, g);
            u32x2_t hl[2];
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) {
                const float p0 = pp[2 * rp], p1 = pp[2 * rp + 1];
                st.pz += p0 * vzf[0][2 * rp] + p1 * vzf[0][2 * rp + 1];
                hl[rp] = split_bf16(p0 * vsf[0][2 * rp], p1 * vsf[0][2 * rp + 1], neg_lo, neg_hi);
            }
            // row j: hi parts of both halves; row j + 8: lo parts
            ahi = u32x4_t{row_swap8_into<0xC>(hl[0][0], hl[0][1]), row_swap8_into<0xC>(hl[1][0], hl[1][1]),
                          row_swap8_into<0x3>(hl[0][1], hl[0][0]), row_swap8_into<0x3>(hl[1][1], hl[1][0])};
            alo = u32x4_t{0u, 0u, 0u, 0u};
        } else {
            float sc[2][4];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[hp][r] = __builtin_fmaf(dq[hp][r], p.score_scale, bias_s);
            float pp[2][4];
            kivi_softmax(st, sc, pp, g, true);

            // P' = p s_t as bf16 hi + lo, and the zero-point sum
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
                for (int rp = 0; rp < 2; ++rp) {
                    const float p0 = pp[hp][2 * rp], p1 = pp[hp][2 * rp + 1];
                    st.pz += p0 * vzf[hp][2 * rp] + p1 * vzf[hp][2 * rp + 1];
                    const u32x2_t hl = split_bf16(p0 * vsf[hp][2 * rp], p1 * vsf[hp][2 * rp + 1], neg_lo, neg_hi);
                    ahi[2 * hp + rp] = hl[0];
                    alo[2 * hp + rp] = hl[1];
                }
            }
        }
        pd.ahi = ahi;
        pd.alo = alo;
#pragma unroll
        for (int hp = 0; hp < kHalves; ++hp)
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) pd.vc[hp][rp] = cb.vc[hp][rp];
    };

    auto back = [&](const Pend& pd) {
        const u32x4_t ahi = pd.ahi, alo = pd.alo;
        // the code offset 128 multiplies exactly the P' the MFMAs consume: sum them
        // with the same MFMAs against ones
        st.pc = mfma_16x16x32_bf16(ahi, kOnes, st.pc);
        if constexpr (!SHARE) st.pc = mfma_16x16x32_bf16(alo, kOnes, st.pc);

        // V: channel 8j + t, tokens 16 hp + 4g + [0, 4) in slots 2 hp + [0, 2)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            u32x4_t bv;
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                for (int rp = 0; rp < 2; ++rp) {
                    // 2 bits: the token half hp sits in bits 2 hp of each 4-bit field
                    const uint32_t w = BITS == 4 ? pd.vc[hp][rp][t >> 2] : pd.vc[0][rp][t >> 2] >> (2 * hp);
                    uint32_t o;
                    switch (t & 3) {
                        case 0: o = v_pair<0>(w, vm0, vm1, vc128); break;
                        case 1: o = v_pair<1>(w, vm0, vm1, vc128); break;
                        case 2: o = v_pair<2>(w, vm0, vm1, vc128); break;
                        default: o = v_pair<3>(w, vm0, vm1, vc128); break;
                    }
                    bv[2 * hp + rp] = o;
                }
            st.acc[t] = mfma_16x16x32_bf16(ahi, bv, st.acc[t]);
            if constexpr (!SHARE) st.acc[t] = mfma_16x16x32_bf16(alo, bv, st.acc[t]);
        }
    };

    // The accumulators hold 128 sum P' on top of the products: fold that
    // offset out every kFoldPages pages, so that the fp32 rounding of a long
    // segment stays relative to 16 pages' offset, not to the whole
    // segment's (4096 pages of 2-bit codes put a 128 / 1.5 times larger
    // offset beside the products and measured 2.5e-3 off the oracle without
    // folding).  It is the epilogue's subtraction, done early.
    auto fold = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int t = 0; t < 8; ++t) st.acc[t][r] = __builtin_fmaf(-128.0f, st.pc[r], st.acc[t][r]);
            st.pc[r] = 0.0f;
        }
    };

    // ---- quantized pages: the loads of the next page are in flight while a
    // page is computed, and page c's back part shares a basic block with page
    // c + 1's front part (independent work to interleave).  The scheduling
    // barriers keep the loads issued before the compute, whose first step (the
    // LDS writes) would otherwise be hoisted above them and wait with nothing
    // in flight.
    if (n_q > 0) {
        KiviBuf b0, b1;
        Pend pd;
        load(b0, 0);
        load(b1, 1);
        __builtin_amdgcn_sched_barrier(0);
        {
            Front F;
            front(b0, F);
            mid(F, b0, pd);
        }
        for (int c = 1; c < n_q;) {
            load(b0, c + 1);
            __builtin_amdgcn_sched_barrier(0);
            {
                Front F;
                front(b1, F);
                back(pd);
                mid(F, b1, pd);
            }
            if (++c >= n_q) break;
            load(b1, c + 1);
            __builtin_amdgcn_sched_barrier(0);
            {
                Front F;
                front(b0, F);
                back(pd);
                mid(F, b0, pd);
            }
            ++c;   // odd here: pages [0, c - 1) are in acc and pc, page c - 1 is pending
            if (((c + 1) & (kFoldPages - 1)) == 0) {
                __asm__ volatile("");
                fold();
            }
        }
        back(pd);
    }

    // ---- fp16 window chunks: tokens nq + 32 (c - pq) + [0, 32).  The odd
    // channels t of the accumulators hold 8x their value (code positions 1 and
    // 3 above), so the window adds 8 p v there.
    const int rfirst = max(page0, pq);
    if (rfirst < page1) {
        u32x4_t qh[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) qh[kb][i] = pack_f16_rne(bf16lo(qb[kb][i]), bf16hi(qb[kb][i]));
        const uint16_t* kw = (const uint16_t*)kp.k_window + ((size_t)b * p.n_kv + h) * kp.window * kHeadDim;
        const uint16_t* vw = (const uint16_t*)kp.v_window + ((size_t)b * p.n_kv + h) * kp.window * kHeadDim;
        for (int c = rfirst; c < page1; ++c) {
            const int rbase = nq + kKiviGroup * (c - pq);
            float sc[2][4];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
                const int pos = rbase + 16 * hp + j;
                u32x4_t kr[4];
                if (pos < len) {
                    const u32x4_t* src = (const u32x4_t*)(kw + (size_t)(pos % kp.window) * kHeadDim + 32 * g);
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) kr[kb] = src[kb];
                } else {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) kr[kb] = u32x4_t{0u, 0u, 0u, 0u};
                }
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) d = mfma_16x16x32_f16(kr[kb], qh[kb], d);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[hp][r] = (rbase + 16 * hp + 4 * g + r < row_end) ? d[r] * p.score_scale : -INFINITY;
            }
            float pp[2][4];
            kivi_softmax(st, sc, pp, g, !SHARE || j < 8);   // lanes 8-15 duplicate heads 0-7 when sharing
            u32x4_t ahi, alo, ahi8, alo8;
            u32x4_t vr[2][4];
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pos = rbase + 16 * hp + 4 * g + r;
                    if (pos < len)
                        vr[hp][r] = *(const u32x4_t*)(vw + (size_t)(pos % kp.window) * kHeadDim + 8 * j);
                    else
                        vr[hp][r] = u32x4_t{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int rp = 0; rp < 2; ++rp) {
                    const float a0 = pp[hp][2 * rp], a1 = pp[hp][2 * rp + 1];
                    const uint32_t hw = pack_f16_rne(a0, a1);
                    ahi[2 * hp + rp] = hw;
                    alo[2 * hp + rp] = pack_f16_rne(a0 - f16_value(hw & 0xFFFFu), a1 - f16_value(hw >> 16));
                    const float b0 = 8.0f * a0, b1 = 8.0f * a1;
                    const uint32_t h8 = pack_f16_rne(b0, b1);
                    ahi8[2 * hp + rp] = h8;
                    alo8[2 * hp + rp] = pack_f16_rne(b0 - f16_value(h8 & 0xFFFFu), b1 - f16_value(h8 >> 16));
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
                u32x4_t bv;
#pragma unroll
                for (int hp = 0; hp < 2; ++hp)
#pragma unroll
                    for (int rp = 0; rp < 2; ++rp)
                        bv[2 * hp + rp] = perm(vr[hp][2 * rp + 1][t >> 1], vr[hp][2 * rp][t >> 1], sel);
                st.acc[t] = mfma_16x16x32_f16((t & 1) ? ahi8 : ahi, bv, st.acc[t]);
                st.acc[t] = mfma_16x16x32_f16((t & 1) ? alo8 : alo, bv, st.acc[t]);
            }
        }
    }

    // ---- epilogue (same output format as the FP8 / INT8 kernel):
    // O = ((acc - 128 pc) / (1 or 8) + sum p z) / l
    float lsum = st.lsum, pz = st.pz;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    pz += __shfl_xor(pz, 16);
    pz += __shfl_xor(pz, 32);
    if constexpr (SHARE) {     // lanes j and j + 8 hold halves of head j's sums
        lsum += bits_to_f32(row_swap8(f32_to_bits(lsum)));
        pz += bits_to_f32(row_swap8(f32_to_bits(pz)));
        // accumulator rows 8-15 (lane groups 2, 3) hold the lo-part products of
        // heads 0-7 (the fp16 window chunks add p = 0 there)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            st.pc[r] += __shfl_xor(st.pc[r], 32);
#pragma unroll
            for (int t = 0; t < 8; ++t) st.acc[t][r] += __shfl_xor(st.acc[t][r], 32);
        }
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
        const float pzh = __shfl(pz, head & 15);
        const float off = 128.0f * st.pc[r];
        if (head < GQ) {
            const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
            f32x4_t o0, o1;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float f = (t & 1) ? 0.125f : 1.0f;
                o0[t] = ((st.acc[t][r] - off) * f + pzh) * inv;
                o1[t] = ((st.acc[t + 4][r] - off) * f + pzh) * inv;
            }
            float* dst = (n_seg == 1)
                             ? p.out + out_row(head) * kHeadDim + 8 * j
                             : p.part_o + (prow0 + head) * kHeadDim + 8 * j;
            *(f32x4_t*)dst = o0;
            *(f32x4_t*)(dst + 4) = o1;
        }
    }
    if (g == 0 && j < GQ) {
        const float l2 = lsum > 0.0f ? st.m_used + __log2f(lsum) : -INFINITY;
        if (n_seg == 1) {
            if (p.lse) p.lse[out_row(j)] = l2 * kLn2;
        } else {
            p.part_lse[prow0 + j] = l2;
        }
    }
}

template <int BITS, bool SHARE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SHARE ? 2 : 1))) void kivi_split_kernel(KiviSplitParams kp) {
    __shared__ __attribute__((aligned(16))) uint8_t s_meta[kSplitThreads / 64][kKiviMetaBytes];
    __shared__ __attribute__((aligned(16))) uint32_t s_zero[64];
    if (threadIdx.x < 64) s_zero[threadIdx.x] = 0u;   // visible after the first barrier below
    const int wid = threadIdx.x >> 6;
    lds_u8* smeta = (lds_u8*)&s_meta[wid][0];
    const lds_u8* szero = (const lds_u8*)&s_zero[0];
    for_each_segment<kKiviGroup>(kp.s, [&](int b, int h, int page0, int page1, int slot, int n_seg, int lane) {
        kivi_segment<BITS, SHARE>(kp, b, h, page0, page1, slot, n_seg, lane, smeta, szero);
    });
}

// rows = query rows per KV head (group x positions): lanes j and j + 8 share a
// row when there are at most 8
static const void* kivi_split_fn(int bits, int rows) {
    if (bits == 2)
        return rows <= 8 ? (const void*)&kivi_split_kernel<2, true> : (const void*)&kivi_split_kernel<2, false>;
    return rows <= 8 ? (const void*)&kivi_split_kernel<4, true> : (const void*)&kivi_split_kernel<4, false>;
}

hipError_t kivi_split_occupancy(int bits, int rows, size_t lds_bytes, int* blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, kivi_split_fn(bits, rows), kSplitThreads,
                                                        lds_bytes);
}

hipError_t launch_kivi_split(const KiviSplitParams& p, int grid, size_t lds_bytes, hipStream_t stream) {
    if (grid <= 0) return hipSuccess;
    KiviSplitParams args = p;
    void* kargs[] = {&args};
    if (p.bits != 4 && p.bits != 2) return hipErrorInvalidValue;
    return hipLaunchKernel(kivi_split_fn(p.bits, p.s.group * p.s.q_len), dim3(grid), dim3(kSplitThreads), kargs, lds_bytes,
                           stream);
}

}  // namespace kvq
