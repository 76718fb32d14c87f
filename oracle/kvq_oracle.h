/*
 * kvq_oracle.h -- CPU oracle for the paged quantized KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * CPU-baseline leg of bench.py may load this library.  The product path (the
 * HIP library) shares no code, header or table with it.
 *
 * Plain C99, fp64 wherever the pages leave the precision open.  The
 * quantizers are encodings: they are written out step by step, in float32
 * where the reading of the pages fixes a float32 operation (scale = amax/448,
 * quotient x/s), and the GPU must reproduce their bytes exactly.
 *
 * Sources (titles of the pages, sections on them):
 *  [molayo]  "KV 캐시 양자화(KV cache quantization): FP8/INT8 K 및 V가 실제로
 *            제공하는 이점과 한계점" (molayo1419.me)
 *  [story]   "KV cache FP8로 동시 요청 76배 수용하기" (storycompiler.tistory.com)
 *  [ryotta]  "KV Cache 압축" (ryotta.opik.net)
 *  [daewooki]"FP8 KV Cache부터 INT4 Weight-Only까지" (daewooki.github.io)
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */
float    kvqo_bf16_value(uint16_t bits);
uint16_t kvqo_bf16_rne(float f);     /* nearest, ties to even mantissa        */
uint16_t kvqo_bf16_up(float f);      /* smallest bf16 >= f (toward +inf)      */
uint16_t kvqo_bf16_down(float f);    /* largest bf16 <= f (toward -inf)       */
double   kvqo_f16_value(uint16_t bits);
uint16_t kvqo_f16_rne(double x);     /* IEEE binary16, nearest-even, subnormals kept */
void     kvqo_bf16_to_f16_array(const uint16_t* bf16, int64_t n, uint16_t* f16);
double   kvqo_e4m3_value(uint8_t code);      /* OCP E4M3 (FN): NaN for 0x7F/0xFF */
uint8_t  kvqo_e4m3_encode(float y);          /* nearest-even, saturating at +-448 */
uint8_t  kvqo_e4m3_encode_f64(double y);     /* the same rule on an exact double */
void     kvqo_e4m3_encode_range(uint32_t first_bits, uint32_t count, uint8_t* codes);
void     kvqo_e4m3_encode_array(const float* y, int64_t n, uint8_t* codes);
double   kvqo_e5m2_value(uint8_t code);      /* OCP E5M2: +-inf at 0x7C/0xFC, NaN for 0x7D-0x7F/0xFD-0xFF */
uint8_t  kvqo_e5m2_encode(float y);          /* nearest-even, saturating at +-57344 */
void     kvqo_e5m2_encode_range(uint32_t first_bits, uint32_t count, uint8_t* codes);
void     kvqo_e5m2_encode_array(const float* y, int64_t n, uint8_t* codes);

/* ---- quantizers: one row of n values ------------------------------------ */
void kvqo_fp8_row(const uint16_t* x_bf16, int n, uint8_t* codes, uint16_t* scale);
void kvqo_fp8_row_static(const uint16_t* x_bf16, int n, uint16_t scale, uint8_t* codes);
void kvqo_int8_row(const uint16_t* x_bf16, int n, uint8_t* codes, uint16_t* scale, uint16_t* zero);
/* generic asymmetric b-bit quantizer over n float32 values read at stride  */
void kvqo_uint_asym(const float* x, int n, int stride, int levels,
                    uint8_t* codes, int code_stride, uint16_t* scale, uint16_t* zero);

/* ---- bulk helpers (OpenMP over rows) ------------------------------------ */
/* dtype 1 = FP8 E4M3, 2 = INT8 asymmetric, 4 = FP8 E5M2.  mode 2 = per-(token,head) scale;
 * mode 0/1 = static scale given per row in static_scale[row].                */
void kvqo_quantize_rows(int dtype, int mode, const uint16_t* x_bf16, int64_t rows, int n,
                        const uint16_t* static_scale, uint8_t* codes, uint16_t* scale,
                        uint16_t* zero);
void kvqo_dequantize_rows(int dtype, int mode, const uint8_t* codes, int64_t rows, int n,
                          const uint16_t* scale, const uint16_t* zero, double* out);

/* KIVI-style b-bit state (bits = 4 or 2) of one (sequence, KV head) stream
 * of T fp16 rows x16[T][n] (fp16 bits).  Tokens [0, nq) are quantized in
 * groups of `group` tokens: K per channel within the group, V per token; the
 * rest stays fp16.  codes: [nq][n] one code per byte (0 .. 2^bits - 1);
 * K: ks/kz [nq/group][n];  V: vs/vz [nq].                                   */
int64_t kvqo_kivi_quantized_count(int64_t T, int resid, int group);
void kvqo_kivi_k(const uint16_t* x16, int64_t nq, int n, int group, int bits,
                 uint8_t* codes, uint16_t* s, uint16_t* z);
void kvqo_kivi_v(const uint16_t* x16, int64_t nq, int n, int bits,
                 uint8_t* codes, uint16_t* s, uint16_t* z);

/* ---- attention (fp64) --------------------------------------------------- */
/* q [n_q][d], k/v [T][n_kv][d] dequantized; out [n_q][d]; lse [n_q] (may be NULL).
 * Query head h reads KV head h / (n_q / n_kv).  T == 0: out = 0, lse = -inf. */
void kvqo_attention(const double* q, const double* k, const double* v, int64_t T,
                    int n_q, int n_kv, int d, double softmax_scale, double* out, double* lse);
/* Score-V product in the FP8 domain (kvq_oracle.c): P per block of `block`
 * tokens relative to the block's integer log2 reference, times the V scale,
 * in E4M3 with a power-of-two block scale.  vcode: V code values without
 * their scale; vs: V scales [T][n_kv].  score_rel: relative score uncertainty
 * of the evaluation the result is compared with (for the allowance only). */
void kvqo_attention_fp8pv(const double* q, const double* k, const double* vcode, const double* vs,
                          int64_t T, int n_q, int n_kv, int d, double softmax_scale, int block,
                          double score_rel, double* out, double* lse, double* allowance);
/* merge P partial results (o [P][d], lse [P]) of disjoint token ranges */
void kvqo_lse_merge(const double* o, const double* lse, int P, int d, double* out, double* lse_out);

/* ---- KV-size accounting ------------------------------------------------- */
double kvqo_kv_bytes(double layers, double n_kv_heads, double head_dim, double seq_len,
                     double batch, double bytes_per_elem);

#ifdef __cplusplus
}
#endif
#endif
