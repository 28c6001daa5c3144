/*
 * oracle.c -- plain, slow CPU oracle for the block-quantized dequant-GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may link, load or call this file; only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark do.  It shares no code,
 * header, table or constant with the GPU path.
 *
 * Sources ("the pages"):
 *   [P1] rustdoc "Module cuda_lane" (qualia_core_db::inference::cuda_lane):
 *        "Functions" list -- q8_0_gemv_oracle_into (decode a row-major GGML
 *        Q8_0 matrix, multiply by x), try_q4k_soa_gemv, try_q4k_soa_qkv (GQA:
 *        K/V only for rows below n_kv), try_q4k_soa_fused_swiglu
 *        (out[i] = silu(gate_row_i . x) * (up_row_i . x)),
 *        try_q4k_soa_ffn_block_residual (out = residual + FFN(x)),
 *        try_cuda_batch_gemv (batch dense GEMM).
 *   [P2] rustdoc source view of weight_cache.rs: doc comment and body of
 *        try_cuda_batch_gemv ("hidden" packed batch x n_in, weight row-major
 *        n_out x n_in, out batch x n_out; dims padded to 16 with zeros and the
 *        result trimmed), and the WeightEntry field comment (rows = out).
 *   [P3] rustdoc "Struct QTensorEngine", method gemm_parity_probe: GPU GEMM and
 *        CPU reference run on the same quantized bytes and input.
 *   The block byte layouts are not printed on the pages; they come from the
 *   workload definitions that accompany them (Q8_0: 34-byte blocks, fp16 d then
 *   32 int8 q, w = d*q; Q4_K: 144-byte super-blocks of 256 weights, fp16 d,
 *   fp16 dmin, 12 bytes of eight 6-bit scales and eight 6-bit mins, 128 bytes of
 *   4-bit q, low nibbles of each 64-element chunk = sub-block 2k, high nibbles =
 *   sub-block 2k+1, w = d*sc*q - dmin*m).  The 6-bit packing itself is not given
 *   anywhere in those sources; the reading used is the public GGML K-quant
 *   layout (see oracle_q4k_unpack_scales).
 *
 * Arithmetic:
 *   - fp16 is decoded from the IEEE 754 binary16 definition.
 *   - Dequantised weights are f32.  Both block formats give products that are
 *     exact in f32 (Q8_0: 11-bit significand x 8-bit integer; Q4_K: d*sc*q and
 *     dmin*m need at most 21 and 17 bits), so the only rounding is Q4_K's final
 *     subtraction, a single IEEE round-to-nearest-even in f32.
 *   - Every dot product accumulates in f64.  A product of two f32 values is
 *     exact in f64; the sum is sequential in j.
 *   - Every dot product also returns S = sum_j |w_ij * x_j| (f64), the scale
 *     the tolerances are stated against.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fPIC -shared (no -ffast-math, no
 * vector intrinsics).  Contraction is off so that (d*sc)*q - dmin*m is
 * evaluated as written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define Q8_0_BYTES 34
#define Q8_0_ELEMS 32
#define Q4K_BYTES 144
#define Q4K_ELEMS 256
#define Q6K_BYTES 210
#define Q6K_ELEMS 256

/* ---------------------------------------------------------------- fp16 -- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   e = 0, f = 0      : signed zero
 *   e = 0, f != 0     : subnormal, value = (-1)^s * f * 2^-24
 *   1 <= e <= 30      : normal,    value = (-1)^s * (1024 + f) * 2^(e - 25)
 *   e = 31, f = 0     : signed infinity
 *   e = 31, f != 0    : NaN (the fraction is carried into the top of the f32
 *                       fraction field)
 * Every finite binary16 value is exactly representable in binary32, so the
 * finite cases below are exact. */
float oracle_fp16_to_f32(uint16_t h)
{
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    float v;
    if (e == 31) {
        uint32_t bits = ((uint32_t)s << 31) | 0x7f800000u | ((uint32_t)f << 13);
        memcpy(&v, &bits, sizeof v);
        return v;
    }
    if (e == 0)
        v = ldexpf((float)f, -24);
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return s ? -v : v;
}

void oracle_fp16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_fp16_to_f32(h[i]);
}

static uint16_t load_le16(const uint8_t* p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* ---------------------------------------------------------------- Q8_0 -- */

/* One row-major GGML Q8_0 matrix, n_out rows of n_in/32 blocks.  Block k of
 * row i starts at byte (i*(n_in/32) + k)*34: bytes 0-1 hold d (fp16, little
 * endian), bytes 2-33 hold q[0..31] as int8.  Weight (i, 32k+t) = d * q[t]. */
void oracle_q8_0_dequantize(const uint8_t* w, int64_t n_in, int64_t n_out, float* out)
{
    const int64_t nb = n_in / Q8_0_ELEMS;
    for (int64_t i = 0; i < n_out; ++i) {
        for (int64_t k = 0; k < nb; ++k) {
            const uint8_t* blk = w + (i * nb + k) * Q8_0_BYTES;
            const float d = oracle_fp16_to_f32(load_le16(blk));
            for (int t = 0; t < Q8_0_ELEMS; ++t) {
                const int8_t q = (int8_t)blk[2 + t];
                out[i * n_in + k * Q8_0_ELEMS + t] = d * (float)q;
            }
        }
    }
}

/* ---------------------------------------------------------------- Q4_K -- */

/* Eight 6-bit scales sc[0..7] and eight 6-bit mins m[0..7] packed into 12
 * bytes s[0..11].  Reading (public GGML K-quant layout; all 96 bits used):
 *   sub-blocks 0..3 : sc[j] = low 6 bits of s[j],   m[j] = low 6 bits of s[j+4]
 *   sub-blocks 4..7 : the low 4 bits come from s[j+4] (sc: low nibble,
 *                     m: high nibble); the high 2 bits are the otherwise unused
 *                     top 2 bits of s[j-4] (sc) and of s[j] (m). */
void oracle_q4k_unpack_scales(const uint8_t* s, uint8_t* sc, uint8_t* m)
{
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        m[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (uint8_t)((s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4));
        m[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
    }
}

/* One row-major GGML Q4_K matrix, n_out rows of n_in/256 super-blocks of 144
 * bytes: d (fp16) at 0, dmin (fp16) at 2, packed scales at 4..15, nibbles
 * qs[0..127] at 16..143.  Element e = 64p + u of the super-block (p = 0..3,
 * u = 0..63) is the low nibble of qs[32p + u] in sub-block 2p when u < 32, and
 * the high nibble of qs[32p + u - 32] in sub-block 2p + 1 otherwise.
 * w = (d*sc)*q - (dmin*m): both products are exact in f32, the subtraction
 * rounds once. */
void oracle_q4k_dequantize(const uint8_t* w, int64_t n_in, int64_t n_out, float* out)
{
    const int64_t nsb = n_in / Q4K_ELEMS;
    for (int64_t i = 0; i < n_out; ++i) {
        for (int64_t k = 0; k < nsb; ++k) {
            const uint8_t* blk = w + (i * nsb + k) * Q4K_BYTES;
            const float d = oracle_fp16_to_f32(load_le16(blk));
            const float dmin = oracle_fp16_to_f32(load_le16(blk + 2));
            uint8_t sc[8], m[8];
            oracle_q4k_unpack_scales(blk + 4, sc, m);
            const uint8_t* qs = blk + 16;
            for (int e = 0; e < Q4K_ELEMS; ++e) {
                const int p = e / 64, u = e % 64;
                int q, sub;
                if (u < 32) {
                    q = qs[32 * p + u] & 0x0f;
                    sub = 2 * p;
                } else {
                    q = qs[32 * p + u - 32] >> 4;
                    sub = 2 * p + 1;
                }
                const float a = (d * (float)sc[sub]) * (float)q;
                const float b = dmin * (float)m[sub];
                out[i * n_in + k * Q4K_ELEMS + e] = a - b;
            }
        }
    }
}

/* Q6_K ([P3] names Q6_K for the embedding and output tensors; no block layout
 * is given there or in the workload definitions, so the reading is the public
 * GGML K-quant layout).  210-byte super-blocks of 256 weights: 128 bytes ql
 * (the low four bits of the 6-bit quants, two per byte), 64 bytes qh (the high
 * two bits, four per byte), 16 int8 scales (one per 16 weights), then fp16 d.
 * Weight e: half h = e / 128, group j = (e % 128) / 32, l = e % 32.  Its low
 * four bits are the low nibble (j = 0, 1) or the high nibble (j = 2, 3) of
 * ql[64h + 32(j % 2) + l]; its high two bits are bits 2j, 2j+1 of
 * qh[32h + l]; its scale is scales[8h + 2j + l / 16]; w = d * sc * (q - 32).
 * d*sc*(q-32) has at most 11 + 7 + 5 significant bits, so it is exact in f32. */
void oracle_q6k_dequantize(const uint8_t* w, int64_t n_in, int64_t n_out, float* out)
{
    const int64_t nsb = n_in / Q6K_ELEMS;
    for (int64_t i = 0; i < n_out; ++i) {
        for (int64_t k = 0; k < nsb; ++k) {
            const uint8_t* blk = w + (i * nsb + k) * Q6K_BYTES;
            const uint8_t* ql = blk;
            const uint8_t* qh = blk + 128;
            const int8_t* sc = (const int8_t*)(blk + 192);
            const float d = oracle_fp16_to_f32(load_le16(blk + 208));
            for (int e = 0; e < Q6K_ELEMS; ++e) {
                const int h = e / 128, j = (e % 128) / 32, l = e % 32;
                const uint8_t lo_byte = ql[64 * h + 32 * (j % 2) + l];
                const int lo = (j < 2) ? (lo_byte & 0x0f) : (lo_byte >> 4);
                const int hi = (qh[32 * h + l] >> (2 * j)) & 3;
                const int q = lo | (hi << 4);
                out[i * n_in + k * Q6K_ELEMS + e] = d * (float)sc[8 * h + 2 * j + l / 16] * (float)(q - 32);
            }
        }
    }
}

/* ------------------------------------------------------ dot products -- */

/* out[b*n_out + i] = sum_j W[i][j] * x[b*n_in + j] in f64, and
 * s_abs[b*n_out + i] = sum_j |W[i][j] * x[b*n_in + j]|, for a dense f32 row
 * block W (n_out x n_in, row-major).  Either output pointer may be NULL. */
static void dense_rows_dot(const float* W, int64_t n_in, int64_t n_out, int64_t batch,
                           const float* x, double* out, double* s_abs)
{
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t i = 0; i < n_out; ++i) {
            double acc = 0.0, sa = 0.0;
            for (int64_t j = 0; j < n_in; ++j) {
                const double p = (double)W[i * n_in + j] * (double)x[b * n_in + j];
                acc += p;
                sa += fabs(p);
            }
            if (out) out[b * n_out + i] = acc;
            if (s_abs) s_abs[b * n_out + i] = sa;
        }
    }
}

typedef void (*dequant_fn)(const uint8_t*, int64_t, int64_t, float*);

/* Dequantise one row at a time (row i's bytes start at i*row_bytes) and dot it
 * with every batch row of x. */
static int quant_rows_dot(dequant_fn deq, int64_t row_bytes, const uint8_t* w, int64_t n_in,
                          int64_t n_out, int64_t batch, const float* x, double* out,
                          double* s_abs)
{
    float* row = (float*)malloc((size_t)n_in * sizeof(float));
    double* o = (double*)malloc((size_t)batch * sizeof(double));
    double* s = (double*)malloc((size_t)batch * sizeof(double));
    if (!row || !o || !s) {
        free(row); free(o); free(s);
        return -1;
    }
    for (int64_t i = 0; i < n_out; ++i) {
        deq(w + i * row_bytes, n_in, 1, row);
        dense_rows_dot(row, n_in, 1, batch, x, o, s);
        for (int64_t b = 0; b < batch; ++b) {
            if (out) out[b * n_out + i] = o[b];
            if (s_abs) s_abs[b * n_out + i] = s[b];
        }
    }
    free(row); free(o); free(s);
    return 0;
}

/* Q8_0 GEMV / batched GEMM: out[b][i] = sum_j deq(W)[i][j] * x[b][j]
 * ([P1] q8_0_gemv_oracle_into; [P2] try_cuda_batch_gemv layouts).  Padding
 * to multiples of 16 adds zero terms only, so it is not modelled. */
int oracle_q8_0_gemv(const uint8_t* w, int64_t n_in, int64_t n_out, int64_t batch,
                     const float* x, double* out, double* s_abs)
{
    return quant_rows_dot(oracle_q8_0_dequantize, (n_in / Q8_0_ELEMS) * Q8_0_BYTES, w, n_in,
                          n_out, batch, x, out, s_abs);
}

/* Q4_K GEMV ([P1] try_q4k_soa_gemv): the same product over Q4_K weights. */
int oracle_q4k_gemv(const uint8_t* w, int64_t n_in, int64_t n_out, int64_t batch,
                    const float* x, double* out, double* s_abs)
{
    return quant_rows_dot(oracle_q4k_dequantize, (n_in / Q4K_ELEMS) * Q4K_BYTES, w, n_in,
                          n_out, batch, x, out, s_abs);
}

/* Dense f32 weights ([P2] try_cuda_batch_gemv): out[b][i] = sum_j W[i][j] x[b][j]. */
/* Q6_K dequant-GEMV ([P1] the GEMV family over another GGML block type; the
 * pages' output and embedding tensors are Q6_K): as oracle_q8_0_gemv. */
int oracle_q6k_gemv(const uint8_t* w, int64_t n_in, int64_t n_out, int64_t batch,
                    const float* x, double* out, double* s_abs)
{
    return quant_rows_dot(oracle_q6k_dequantize, (n_in / Q6K_ELEMS) * Q6K_BYTES, w, n_in,
                          n_out, batch, x, out, s_abs);
}

int oracle_f32_gemm(const float* w, int64_t n_in, int64_t n_out, int64_t batch,
                    const float* x, double* out, double* s_abs)
{
    dense_rows_dot(w, n_in, n_out, batch, x, out, s_abs);
    return 0;
}

/* Down-projection with residual ([P1] try_q4k_soa_ffn_block_residual):
 * out[b][i] = residual[b][i] + sum_j deq(W)[i][j] x[b][j].  s_abs is the S of
 * the dot product alone. */
int oracle_q8_0_gemv_residual(const uint8_t* w, int64_t n_in, int64_t n_out, int64_t batch,
                              const float* x, const float* residual, double* out,
                              double* s_abs)
{
    if (oracle_q8_0_gemv(w, n_in, n_out, batch, x, out, s_abs) != 0) return -1;
    for (int64_t k = 0; k < batch * n_out; ++k)
        out[k] += (double)residual[k];
    return 0;
}

/* Fused QKV with GQA ([P1] try_q4k_soa_qkv): three independent products that
 * share x; Q has n_q rows, K and V have n_kv rows each. */
int oracle_q8_0_qkv(const uint8_t* wq, const uint8_t* wk, const uint8_t* wv, int64_t n_in,
                    int64_t n_q, int64_t n_kv, int64_t batch, const float* x, double* q_out,
                    double* k_out, double* v_out, double* sq, double* sk, double* sv)
{
    if (oracle_q8_0_gemv(wq, n_in, n_q, batch, x, q_out, sq) != 0) return -1;
    if (oracle_q8_0_gemv(wk, n_in, n_kv, batch, x, k_out, sk) != 0) return -1;
    if (oracle_q8_0_gemv(wv, n_in, n_kv, batch, x, v_out, sv) != 0) return -1;
    return 0;
}

/* silu(z) = z * sigmoid(z) = z / (1 + exp(-z)).  The pages use the name only;
 * this is the standard definition.  For z below about -709 exp(-z) is +inf and
 * the quotient is -0, the limit. */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* Fused SwiGLU ([P1] try_q4k_soa_fused_swiglu):
 * out[b][i] = silu(g) * u with g = gate_row_i . x_b and u = up_row_i . x_b.
 * g, u, and their S values (sg, su) are returned too when non-NULL. */
int oracle_q8_0_swiglu(const uint8_t* w_gate, const uint8_t* w_up, int64_t n_in, int64_t n_out,
                       int64_t batch, const float* x, double* out, double* g, double* u,
                       double* sg, double* su)
{
    const size_t n = (size_t)(batch * n_out);
    double* gg = (double*)malloc(n * sizeof(double));
    double* uu = (double*)malloc(n * sizeof(double));
    if (!gg || !uu) {
        free(gg); free(uu);
        return -1;
    }
    int rc = oracle_q8_0_gemv(w_gate, n_in, n_out, batch, x, gg, sg);
    if (rc == 0) rc = oracle_q8_0_gemv(w_up, n_in, n_out, batch, x, uu, su);
    if (rc == 0) {
        for (size_t k = 0; k < n; ++k) {
            if (out) out[k] = oracle_silu(gg[k]) * uu[k];
            if (g) g[k] = gg[k];
            if (u) u[k] = uu[k];
        }
    }
    free(gg); free(uu);
    return rc;
}

/* ---------------------------------------------------------------- top-k -- */

/* Vocabulary top-k ([P3] dispatch_output_topk_chunked, and
 * dispatch_output_top1_chunked for k = 1): the k largest logits of each batch
 * row with their vocabulary ids, largest first.  The pages fix no order among
 * equal logits; the reading used is "equal values by smaller index", so top-1
 * is the first maximum (the usual argmax convention).  Values compare
 * numerically, so -0 and +0 are equal; NaN has no place in that order and is
 * rejected.  Written as a plain sort of (value, index) pairs with the C
 * library's qsort, then the first k. */
typedef struct {
    float v;
    int64_t i;
} topk_item;

static int topk_cmp(const void* pa, const void* pb)
{
    const topk_item* a = (const topk_item*)pa;
    const topk_item* b = (const topk_item*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

int oracle_topk(const float* v, int64_t n, int64_t batch, int64_t k, int32_t* idx, float* val)
{
    if (n < 1 || batch < 1 || k < 1 || k > n || n > INT32_MAX) return -1;
    topk_item* it = (topk_item*)malloc((size_t)n * sizeof(topk_item));
    if (!it) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t i = 0; i < n; ++i) {
            const float f = v[b * n + i];
            if (isnan(f)) {
                free(it);
                return -1;
            }
            it[i].v = f;
            it[i].i = i;
        }
        qsort(it, (size_t)n, sizeof(topk_item), topk_cmp);
        for (int64_t r = 0; r < k; ++r) {
            idx[b * k + r] = (int32_t)it[r].i;
            val[b * k + r] = it[r].v;
        }
    }
    free(it);
    return 0;
}

/* -------------------------------------------------------------- RMSNorm -- */

/* RMSNorm ([P3] apply_output_norm_inplace: the output_norm of a pre-norm model,
 * applied before the vocabulary projection; the same normalisation precedes a
 * block's attention and FFN products).  The pages print no formula; the usual
 * definition is used, in f64:
 *   out[b][j] = x[b][j] / sqrt(mean_j x[b][j]^2 + eps) * w[j]. */
int oracle_rmsnorm(const float* x, int64_t n, int64_t batch, const float* w, double eps, double* out)
{
    if (n < 1 || batch < 1 || !(eps >= 0.0)) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        double ss = 0.0;
        for (int64_t j = 0; j < n; ++j) ss += (double)x[b * n + j] * (double)x[b * n + j];
        const double r = 1.0 / sqrt(ss / (double)n + eps);
        for (int64_t j = 0; j < n; ++j) out[b * n + j] = (double)x[b * n + j] * r * (double)w[j];
    }
    return 0;
}

/* ------------------------------------------------------ decode attention -- */

/* Device decode attention ([P1] try_q4k_soa_attention_device: rotary position
 * embedding of the new q and k, append of k and v to the device KV cache, GQA
 * scaled dot-product attention; the O projection that follows is a GEMV with
 * residual).  The pages name these steps and keep an f32 KV cache, but print
 * no formula; the readings used:
 *   - RoPE on adjacent pairs: pair i = (x[2i], x[2i+1]) of a head of even
 *     length d rotates by angle pos * base^(-2i/d):
 *       (a, b) -> (a cos - b sin, a sin + b cos);
 *   - cache layout [kv_head][max_seq][d], f32, position pos written in place;
 *   - GQA: q head h reads kv head h / (n_head / n_kv_head);
 *   - scores s_t = scale * (q_h . K[t]) for t < n_ctx, p = softmax(s),
 *     out_h = sum_t p_t V[t].
 * Everything in f64 here.  oracle_rope rotates in place; oracle_attention
 * also returns A[h][j] = sum_t p_t |V[t][j]|, the scale of its tolerance. */
void oracle_rope(double* x, int64_t n_heads, int64_t d, int64_t pos, double base)
{
    for (int64_t h = 0; h < n_heads; ++h) {
        for (int64_t i = 0; i < d / 2; ++i) {
            const double ang = (double)pos * pow(base, -2.0 * (double)i / (double)d);
            const double c = cos(ang), s = sin(ang);
            const double a = x[h * d + 2 * i], b = x[h * d + 2 * i + 1];
            x[h * d + 2 * i] = a * c - b * s;
            x[h * d + 2 * i + 1] = a * s + b * c;
        }
    }
}

int oracle_attention(const double* q, const float* k_cache, const float* v_cache, int64_t n_head,
                     int64_t n_kv, int64_t d, int64_t n_ctx, int64_t max_seq, double scale,
                     double* out, double* a_abs)
{
    if (n_head < 1 || n_kv < 1 || n_head % n_kv != 0 || d < 2 || n_ctx < 1 || n_ctx > max_seq) return -1;
    double* s = (double*)malloc((size_t)n_ctx * sizeof(double));
    if (!s) return -1;
    const int64_t group = n_head / n_kv;
    for (int64_t h = 0; h < n_head; ++h) {
        const int64_t kv = h / group;
        const float* K = k_cache + kv * max_seq * d;
        const float* V = v_cache + kv * max_seq * d;
        double m = -INFINITY;
        for (int64_t t = 0; t < n_ctx; ++t) {
            double dot = 0.0;
            for (int64_t j = 0; j < d; ++j) dot += q[h * d + j] * (double)K[t * d + j];
            s[t] = scale * dot;
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < n_ctx; ++t) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        for (int64_t j = 0; j < d; ++j) {
            double o = 0.0, a = 0.0;
            for (int64_t t = 0; t < n_ctx; ++t) {
                o += s[t] * (double)V[t * d + j];
                a += s[t] * fabs((double)V[t * d + j]);
            }
            out[h * d + j] = o / l;
            if (a_abs) a_abs[h * d + j] = a / l;
        }
    }
    free(s);
    return 0;
}
