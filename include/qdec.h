/*
 * qdec.h -- C ABI of libqdec, block-quantized dequant-GEMV/GEMM for AMD MI355X
 * (gfx950).
 *
 * Operations follow three rustdoc pages of the qualia_core_db crate:
 *   [cuda_lane]    "Module cuda_lane" (inference::cuda_lane), Functions and
 *                  Constants sections;
 *   [weight_cache] the source view of inference/cuda_lane/weight_cache.rs
 *                  (try_cuda_batch_gemv and the cache functions);
 *   [QTensorEngine] "Struct QTensorEngine" (gguf_bridge), its methods.
 * The GGML block layouts are not printed on those pages; the ones used are the
 * workload definitions that accompany them:
 *   Q8_0: 34-byte blocks of 32 weights = fp16 d (little-endian) then 32 int8 q;
 *         w = d*q.
 *   Q4_K: 144-byte super-blocks of 256 weights = fp16 d, fp16 dmin, 12 bytes of
 *         eight 6-bit scales and eight 6-bit mins (GGML K-quant packing), 128
 *         bytes of nibbles (low nibbles of each 64-element chunk p = sub-block
 *         2p, high nibbles = sub-block 2p+1); w = d*sc*q - dmin*m.
 *   Q6_K: named by [QTensorEngine] (embedding and output tensors) without a
 *         layout; the public GGML K-quant layout is used: 210-byte super-blocks
 *         of 256 weights = ql[128] (low 4 bits), qh[64] (high 2 bits), int8
 *         scales[16], fp16 d; weight 128h + 32j + l takes the low (j < 2) or
 *         high nibble of ql[64h + 32(j%2) + l], bits 2j..2j+1 of qh[32h + l]
 *         and scales[8h + 2j + l/16]; w = d*scale*(q - 32).
 *
 * Conventions for every call below
 *   - Weights are GGML raw block bytes in DEVICE memory, row-major: row i of an
 *     n_out x n_in matrix starts at byte i*(n_in/32)*34 (Q8_0) or
 *     i*(n_in/256)*144 (Q4_K) ("rows = out", [weight_cache] WeightEntry).
 *   - x is DEVICE f32, packed batch x n_in; out is DEVICE f32, packed
 *     batch x n_out ([weight_cache] try_cuda_batch_gemv doc comment):
 *     out[b*n_out + i] = sum_j deq(W)[i][j] * x[b*n_in + j].
 *   - Every call is asynchronous and ordered on `stream` (0 = the null stream).
 *     Nothing is read back; faults inside kernels surface at the caller's next
 *     synchronisation, as usual for HIP.
 *   - The caller owns w, x, out and residual and keeps them alive until the
 *     stream has passed the call.  out must not overlap x or the weights
 *     (aliasing residual is allowed where stated).
 *   - Repacked weights: the first use of a weight pointer (or qdec_prepare)
 *     copies its blocks once into a library-owned, aligned device layout
 *     ("Call once at plan build", [cuda_lane] preload_q4k_soa_weights).  The
 *     copy is keyed by (device, pointer, type, n_in, n_out); the caller promises
 *     that the bytes behind a cached pointer do not change until qdec_release
 *     or qdec_clear_cache ("immutable", [cuda_lane] preload_resident_blob).
 *     Inside HIP stream capture no copy can be made or waited for
 *     (QDEC_EINVAL): call qdec_prepare, which returns once the copy is
 *     complete, for every weight before capturing.
 *   - Workspace: the matrix-core GEMV for 3..8 batch rows (Q8_0, n_in a
 *     multiple of 256 up to 8192) keeps the sums of its K slices where it
 *     splits K over workgroups (never at n_in 1024, 2048, 3072 or 4096,
 *     nor at 6144 or 8192 with up to 4 rows outside SwiGLU, whose rows stay
 *     in one workgroup), q8_0_gemv_topk keeps its candidate lists,
 *     attention keeps its chunk partials, and the batched GEMMs on their
 *     DMA-fed path (n_in % 64 == 0, and even n_out for Q8_0; K split over up
 *     to 8 slices when the output has few 128 x 128 tiles) round x to bf16
 *     and keep the slices' partial products (as do both batched GEMMs on
 *     their other K-split shapes), in a library-owned device buffer, one per
 *     (device, stream), made (or grown) on the first such call on that stream
 *     and freed by qdec_clear_cache.  Calls on one stream share it in
 *     stream order; calls on different streams never share one.  When a
 *     stream's buffer grows, the old one is kept (not freed) until
 *     qdec_clear_cache, because a graph captured earlier may still use it.  A stream
 *     capture cannot allocate it, so a capture on a stream that has none takes
 *     the VALU kernels (same results to the f32 tolerance), or for the GEMMs
 *     the register-staged kernel with its K slices added by f32 atomics (same
 *     products; the order of the slice sums, and so the last bits, can vary).
 *   - Return value: QDEC_OK (0) or a negative qdec_status.  Invalid arguments
 *     are rejected with QDEC_EINVAL before any HIP call; a failed allocation
 *     returns QDEC_ENOMEM; a failed launch or HIP call returns QDEC_EHIP.
 *     The library never falls back to a CPU path.  qdec_last_error() describes
 *     the last failure on the calling thread.
 *   - Thread safety: calls may come from several host threads; the repack
 *     cache is guarded by a mutex.
 *   - Environment (debugging only): QDEC_LOG=1 writes one stderr line per
 *     library allocation or release ("qdec|repack|...", "qdec|workspace|...",
 *     "qdec|release|...", "qdec|clear_cache|...": device, pointer, type,
 *     shape, bytes); QDEC_FAIL_ALLOC=1 makes every repack or workspace
 *     allocation fail with QDEC_ENOMEM.
 */
#ifndef QDEC_H
#define QDEC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(QDEC_BUILDING)
#define QDEC_API __attribute__((visibility("default")))
#else
#define QDEC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QDEC_OK = 0,
    QDEC_EINVAL = -1,        /* bad dimension, null pointer, batch out of range */
    QDEC_ENOMEM = -2,        /* device allocation for a repacked copy failed */
    QDEC_EHIP = -3,          /* a HIP runtime call or kernel launch failed */
    QDEC_EUNSUPPORTED = -4   /* no kernel for this device or shape */
} qdec_status;

/* GGML type ids (F32: dense f32 weights, for qdec_prepare only). */
typedef enum { QDEC_TYPE_F32 = 0, QDEC_TYPE_Q8_0 = 8, QDEC_TYPE_Q4_K = 12, QDEC_TYPE_Q6_K = 14 } qdec_type;

/* Largest batch accepted by the GEMV-shaped calls (decode).  The batched GEMM
 * calls take any batch >= 1. */
#define QDEC_GEMV_MAX_BATCH 8

/* ------------------------------------------------------------ compute -- */

/* Q8_0 dequant-GEMV ([cuda_lane] try_q8_0_cuda_gemv, q8_0_gemv_oracle_into):
 * out[b][i] = sum_j deq(W)[i][j] * x[b][j] for 1 <= batch <= 8.
 * n_in % 32 == 0, n_in, n_out >= 1.  f32 accumulation.  Reproducibility: the
 * same inputs give the same bits on every call on a given path (with 3..8
 * batch rows at n_in 1024, 2048, 3072 or 4096, and 3..4 rows at 6144 or
 * 8192, each row stays in one workgroup; otherwise K is split over
 * workgroups unless the grid is large enough without it, and a further small
 * launch adds the slices' sums in a fixed order).  On the one-workgroup
 * shapes x enters the matrix cores as a 30-bit fixed-point number per
 * 32-value block (error at most 2^-29 of the block's largest |x| per value,
 * beyond f32 rounding) and a non-finite x makes every output of its batch
 * row NaN. */
QDEC_API int q8_0_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
              const float* x, float* out, hipStream_t stream);

/* Down-projection with residual ([cuda_lane] try_q4k_soa_ffn_block_residual):
 * out[b][i] = residual[b][i] + sum_j deq(W)[i][j] * x[b][j].
 * residual is device f32 batch x n_out; out may be the same buffer as
 * residual (in-place update); residual must not overlap x (QDEC_EINVAL).
 * Other conditions as q8_0_gemv. */
QDEC_API int q8_0_gemv_residual(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
                       const float* x, const float* residual, float* out,
                       hipStream_t stream);

/* Fused QKV with GQA ([cuda_lane] try_q4k_soa_qkv): one launch computes
 * q = Wq x (n_q rows), k = Wk x and v = Wv x (n_kv rows each) from one shared
 * x.  q_out is batch x n_q, k_out and v_out are batch x n_kv, three separate
 * device buffers.  1 <= n_kv <= n_q; other conditions as q8_0_gemv. */
QDEC_API int q8_0_qkv(const void* wq, const void* wk, const void* wv, int64_t n_in,
             int64_t n_q, int64_t n_kv, int64_t batch, const float* x,
             float* q_out, float* k_out, float* v_out, hipStream_t stream);

/* Fused SwiGLU expansion ([cuda_lane] try_q4k_soa_fused_swiglu):
 * out[b][i] = silu(g) * u, g = gate_row_i . x_b, u = up_row_i . x_b,
 * silu(z) = z / (1 + exp(-z)).  Both weights are n_out x n_in Q8_0.
 * Conditions as q8_0_gemv. */
QDEC_API int q8_0_swiglu(const void* w_gate, const void* w_up, int64_t n_in, int64_t n_out,
                int64_t batch, const float* x, float* out, hipStream_t stream);

/* Largest k of q8_0_gemv_topk. */
#define QDEC_TOPK_MAX 256

/* Vocabulary projection with on-device top-k ([QTensorEngine]
 * dispatch_output_topk_chunked, and dispatch_output_top1_chunked for k = 1):
 * logits = W x exactly as q8_0_gemv computes them (same kernels, same bits),
 * written to `logits` (device f32, batch x n_out, kept for a sampler), then,
 * per batch row, the k largest logits: top_idx[b*k + r] (int32 vocabulary row)
 * and top_val[b*k + r] = logits[b*n_out + top_idx[b*k + r]], r = 0 first.
 * Order: larger logit first; equal logits by smaller index; -0 equals +0
 * (NaN logits, possible only from non-finite inputs, rank by bit pattern).
 * 1 <= k <= min(n_out, QDEC_TOPK_MAX); other conditions as q8_0_gemv.  The
 * selection takes two launches: one workgroup per 2048 logits (4096 or 8192
 * when n_out * k is large) keeps its chunk's k largest, then one workgroup per
 * row merges the row's lists.  The lists live in the stream's workspace (see
 * Conventions; batch * chunks * k * 8 bytes): a capturing stream must already
 * hold one that large (make the same call on it once before capturing), else
 * QDEC_EINVAL.  When ceil(n_out / 8192) * k exceeds 16384 a staged selection
 * of more launches runs instead.  logits, top_idx, top_val and x must not
 * overlap. */
QDEC_API int q8_0_gemv_topk(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
                   const float* x, int64_t k, float* logits, int32_t* top_idx,
                   float* top_val, hipStream_t stream);

/* Allocation-free variant of q8_0_gemv_topk, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and kernels as
 * q8_0_gemv_topk (same logits bits and the same top_idx/top_val), but it calls
 * no hipMalloc, hipFree or other allocating routine:
 *   - w must already have its repacked copies (qdec_prepare), else QDEC_EINVAL;
 *   - its scratch (the K slices' sums of the 3..8-row matrix-core
 *     projection where it splits K, then the top-k candidate lists) is one
 *     static device array of QDEC_NOALLOC_SCRATCH_BYTES per GPU, held until
 *     the process ends; calls needing more (large batch x k x n_out, or
 *     3..8 rows of a wide n_in) are rejected with QDEC_EINVAL before any
 *     launch.  128256 logits of n_in <= 3072 fit for every batch and k.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (on different streams, or from different host threads) race and
 * must not be made; calls ordered on one stream are safe.  Nothing carries
 * over from one call to the next (every scratch byte read is written first
 * in the same call). */
#define QDEC_NOALLOC_SCRATCH_BYTES (16 << 20)
QDEC_API int q8_0_gemv_topk_noalloc(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
                                    const float* x, int64_t k, float* logits, int32_t* top_idx,
                                    float* top_val, hipStream_t stream);

/* RMSNorm ([QTensorEngine] apply_output_norm_inplace, the pre-norm model's
 * output_norm; the pages give no formula, the usual one is used):
 * out[b][j] = x[b][j] / sqrt(mean_j x[b][j]^2 + eps) * w[j], any batch >= 1
 * and n >= 1, 0 <= eps <= 1; the sum of squares and the root are taken in f64
 * (no overflow for any f32 row), the products in f32.  out may be x (in place) but must not
 * overlap it otherwise.  x, w, out are device f32. */
QDEC_API int qdec_rmsnorm(const float* x, int64_t n, int64_t batch, const float* w, float eps,
                 float* out, hipStream_t stream);

/* Attention input of a pre-norm decode block: (q, k, v) = QKV(RMSNorm(h;
 * norm_w, eps)) as q8_0_qkv over the normalised rows ([cuda_lane]
 * try_q4k_soa_qkv, [QTensorEngine] dispatch_transformer_layer).  One batch row
 * at n_in a multiple of 1024 (up to 16384) folds the norm into the product:
 * out = r * (W (norm_w * h)), r = 1/sqrt(mean h^2 + eps), one launch, scratch
 * unused (may be NULL).  Otherwise h is normalised into scratch (device f32,
 * batch x n_in, 16-byte aligned) first.  norm_w: device f32 n_in, 16-byte
 * aligned.  Other conditions as q8_0_qkv. */
QDEC_API int q8_0_rmsnorm_qkv(const void* wq, const void* wk, const void* wv, int64_t n_in,
                     int64_t n_q, int64_t n_kv, int64_t batch, const float* h,
                     const float* norm_w, float eps, float* q_out, float* k_out,
                     float* v_out, float* scratch, hipStream_t stream);

/* The rest of a pre-norm decode block once attention has produced `attn`
 * (batch x n_q; the attention core itself -- RoPE, KV cache, softmax -- is
 * not part of this library):
 *   h <- h + Wo attn                          (Wo: n_embd x n_q)
 *   f  = SwiGLU(RMSNorm(h; ffn_norm, eps))    (gate, up: n_ff x n_embd)
 *   h <- h + Wd f                             (Wd: n_embd x n_ff)
 * three launches at one batch row (the norm folded into the SwiGLU product),
 * four otherwise ([QTensorEngine] dispatch_transformer_layer,
 * [cuda_lane] try_q4k_soa_fused_swiglu and try_q4k_soa_ffn_block_residual).
 * h: device f32 batch x n_embd, updated in place.  scratch: device f32 of
 * batch x (n_ff + n_embd) floats, 16-byte aligned, not overlapping h or attn
 * (f, then the normalised h).  n_q, n_embd, n_ff multiples of 32;
 * 1 <= batch <= 8. */
QDEC_API int q8_0_attn_out_ffn(const void* wo, const void* w_gate, const void* w_up,
                      const void* w_down, int64_t n_embd, int64_t n_q, int64_t n_ff,
                      int64_t batch, float* h, const float* attn, const float* ffn_norm,
                      float eps, float* scratch, hipStream_t stream);

/* Decode attention for one new token ([cuda_lane]
 * try_q4k_soa_attention_device: RoPE, device KV append, GQA scaled
 * dot-product attention; the O projection after it is q8_0_gemv_residual or
 * q8_0_attn_out_ffn).  The pages give no formulas; the ones used:
 *   RoPE: adjacent pairs (x[2i], x[2i+1]) of each head rotate by the angle
 *         pos * base^(-2i/head_dim): (a, b) -> (a cos - b sin, a sin + b cos),
 *         computed in f64 and rounded once to f32;
 *   KV cache: device f32 [n_kv][max_seq][head_dim] for K and for V;
 *   GQA: query head h reads kv head h / (n_head / n_kv);
 *   attention: out_h = sum_{t < n_ctx} softmax_t(scale * q_h . K[t]) V[t].
 * head_dim 64 or 128; n_kv divides n_head with at most 16 query heads per kv
 * head.  q (n_head x head_dim), k, v (n_kv x head_dim) are device f32. */

/* Rotate q and k in place for position pos (0 <= pos < max_seq) and write the
 * rotated k and v at position pos of the caches.  base > 1 (e.g. 10000 or
 * 500000).  No buffers may overlap. */
QDEC_API int qdec_rope_kv_append(float* q, float* k, const float* v, int64_t n_head,
                        int64_t n_kv, int64_t head_dim, int64_t pos, float base, float* k_cache,
                        float* v_cache, int64_t max_seq, hipStream_t stream);

/* out (n_head x head_dim, device f32) = attention of q over positions
 * 0 .. n_ctx-1 (1 <= n_ctx <= max_seq), scale > 0 (usually 1/sqrt(head_dim)).
 * f32 dot products and sums, expf; with n_ctx > 128 the per-chunk partials
 * (n_head * ceil(n_ctx/128) * (head_dim + 2) floats) live in the stream's
 * workspace: a capturing stream must already hold one (make one call on it
 * before capturing), else QDEC_EINVAL.  out must not overlap the inputs. */
QDEC_API int qdec_attention_decode(const float* q, const float* k_cache, const float* v_cache,
                          int64_t n_head, int64_t n_kv, int64_t head_dim, int64_t n_ctx,
                          int64_t max_seq, float scale, float* out, hipStream_t stream);

/* Q4_K dequant-GEMV ([cuda_lane] try_q4k_soa_gemv): as q8_0_gemv over Q4_K
 * weights; n_in % 256 == 0, 1 <= batch <= 8.  With n_in one of 1024, 2048,
 * 3072, 4096, 6144, 8192 the product runs on the integer matrix cores (5..8
 * rows at 6144 and 8192 as two launches of 2..4 rows each; a captured graph
 * then holds both) from a second, fragment-tiled copy of the weight (made
 * on first use and by qdec_prepare, the same 148 bytes per 256 weights; a
 * graph captured before that copy exists runs the vector kernel instead).
 * That path takes x as a
 * 30-bit fixed-point number per 32 values: a value below 2^-6 of its group's
 * largest |x| keeps its bits down to 2^-29 of that largest value only, which
 * adds at most 2^-29 max|x| sum_k |d sc q_k| per output; a NaN or infinity in
 * x makes the outputs NaN or infinite (with 2..8 batch rows: every output of
 * that batch row NaN). */
QDEC_API int q4k_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
             const float* x, float* out, hipStream_t stream);

/* Q6_K dequant-GEMV (the GEMV family of [cuda_lane] over the Q6_K blocks
 * that [QTensorEngine] uses for the output and embedding tensors): as
 * q8_0_gemv over Q6_K weights; n_in % 256 == 0, 1 <= batch <= 8.  Products
 * are exact (each weight is an integer times an exact scale), f32 sums.  With
 * n_in one of 1024, 2048, 3072, 4096, 6144, 8192 every batch runs on the
 * integer matrix cores (one launch while the batch, rounded up to 2, 4 or 8,
 * times n_in is at most 32768; 5..8 rows at 6144 and 8192 as two launches)
 * from a second, fragment-tiled copy of the weight (made
 * on first use and by qdec_prepare, 210 bytes per 256 weights; a graph
 * captured before that copy exists runs the vector kernel instead).  That
 * path takes x as a 30-bit fixed-point number per 16 values (one scale
 * group), which adds at most 2^-29 max|x| of the group per value, and a NaN
 * or infinity in x makes every output of its batch row NaN. */
QDEC_API int q6k_gemv(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
             const float* x, float* out, hipStream_t stream);

/* Batched prefill-shaped GEMM over Q8_0 weights ([weight_cache]
 * try_cuda_batch_gemv: C[m x n] = A[m x k] B[k x n] with m = batch,
 * k = n_in, n = n_out, B = W transposed).  Dequantised weight tiles and x
 * tiles are rounded to bf16 and contracted on MFMA with f32 accumulation
 * (relative error bound about 4e-3 of sum_j |w_ij x_bj|).  Any batch >= 1;
 * n_in % 32 == 0.  The pages' padding to multiples of 16 adds zero terms
 * only and is handled inside the kernel. */
QDEC_API int q8_0_gemm_batched(const void* w, int64_t n_in, int64_t n_out, int64_t batch,
                      const float* x, float* out, hipStream_t stream);

/* The same contraction over dense f32 row-major weights (n_out x n_in, device
 * memory), bf16 MFMA with f32 accumulation: both operands rounded to bf16
 * (round to nearest even), as in q8_0_gemm_batched.  Any batch >= 1,
 * n_in % 32 == 0.  By default W is read in place and rounded as it is loaded.
 * After qdec_prepare(w, QDEC_TYPE_F32, ...) the call reads the library's bf16
 * copy of W instead (n_in * n_out * 2 bytes, same rounding, so the same
 * products; with n_in % 64 == 0 the DMA-fed kernel of q8_0_gemm_batched runs
 * on it); the copy is never made implicitly, and once it exists W must not
 * change until qdec_release. */
QDEC_API int f32_gemm_batched(const float* w, int64_t n_in, int64_t n_out, int64_t batch,
                     const float* x, float* out, hipStream_t stream);

/* -------------------------------------------------------- repack cache -- */

/* Repack w now (load time, not timed), type QDEC_TYPE_Q8_0, QDEC_TYPE_Q4_K or QDEC_TYPE_Q6_K
 * ([cuda_lane] preload_q4k_soa_weights), and wait on the host until the copy
 * is complete.  Idempotent.  QDEC_TYPE_F32 (w: dense f32, n_in % 32 == 0,
 * 16-byte aligned) makes the bf16 copy f32_gemm_batched then reads. */
QDEC_API int qdec_prepare(const void* w, int type, int64_t n_in, int64_t n_out, hipStream_t stream);

/* Free every repacked copy made from w (all types and shapes) on the current
 * device.  Returns QDEC_EINVAL if there was none.  Waits for the device.
 * A HIP graph captured from calls on w reads these copies: after this call
 * such a graph must not be replayed again (capture it anew). */
QDEC_API int qdec_release(const void* w);

/* Free every repacked copy and every workspace on every device ([cuda_lane]
 * clear_weight_cache, "tests / model swap").  Waits for the devices.  Every
 * graph captured from library calls is invalid afterwards (it holds the
 * addresses of copies and workspaces); capture again after new calls. */
QDEC_API void qdec_clear_cache(void);

/* Number of repacked copies currently held ([cuda_lane] weight_cache_len). */
QDEC_API int64_t qdec_cache_len(void);

/* ----------------------------------------------- dequantisation exports -- */

/* Write deq(W) as device f32, n_out x n_in row-major, from the same repacked
 * copy the compute calls read.  Bit-exact with the block definition: Q8_0
 * products are exact in f32; Q4_K rounds once, in the final subtraction. */
QDEC_API int q8_0_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream);
QDEC_API int q4k_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream);
/* Q6_K: d*scale*(q - 32) has at most 23 significant bits, exact in f32. */
QDEC_API int q6k_dequantize(const void* w, int64_t n_in, int64_t n_out, float* out, hipStream_t stream);

/* ---------------------------------------------------------- diagnostics -- */

/* Text of the last failure on this thread ("" if none).  Owned by the library,
 * valid until the next call on the same thread. */
QDEC_API const char* qdec_last_error(void);

/* Number of kernels the library has launched in this process (a witness that
 * the GPU path ran; [QTensorEngine] gemm_parity_probe). */
QDEC_API uint64_t qdec_launch_count(void);

/* Host-side extent check, no device needed: for an n_out x n_in product at
 * `batch` rows, work out every launch plan the library would choose (the
 * 3..8-row matrix-core GEMV in its plain, residual, SwiGLU and QKV forms;
 * the batched GEMMs on Q8_0 weights and on dense f32 weights with and
 * without their bf16 copy, each with and without a workspace) and check that
 * the last element each kernel instance reads or writes lies inside the
 * buffers it is given (weights, x, workspace).  The launchers run the same
 * checks and refuse a failing plan.  QDEC_OK, QDEC_EINVAL for invalid
 * dimensions (n_in % 32 != 0, ...), QDEC_EUNSUPPORTED naming the overrun
 * otherwise (a library bug). */
QDEC_API int qdec_check_plans(int64_t n_in, int64_t n_out, int64_t batch);

/* One empty kernel on `stream` (launch-latency probe, the analogue of
 * [QTensorEngine] bench_empty_submit_roundtrip). */
QDEC_API int qdec_empty_kernel(hipStream_t stream);

/* Plain device copy of `bytes` bytes (bytes % 16 == 0, both pointers 16-byte
 * aligned): the known-size reference kernel for HBM byte counters. */
QDEC_API int qdec_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

/* Plain streaming read of `bytes` bytes of device memory at src (bytes % 16
 * == 0, src 16-byte aligned): each lane issues loads_per_lane (1, 2, 4, 8 or
 * 16) non-temporal 16-byte loads before using any of them, a workgroup of 256
 * lanes covering 4 KB * loads_per_lane contiguous bytes.  The HBM read
 * ceiling the weight-streaming kernels are compared with: a measurement
 * probe beside qdec_empty_kernel (the pages time only an empty submit,
 * [QTensorEngine] bench_empty_submit_roundtrip; no operation of theirs
 * corresponds to it).  sink: device
 * memory of at least 4 bytes, not overlapping src, written only if the XOR
 * of a lane's loaded words equals a fixed constant (its contents carry no
 * meaning; the write keeps the loads from being removed). */
QDEC_API int qdec_stream_read(const void* src, int64_t bytes, int loads_per_lane, uint32_t* sink,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QDEC_H */
