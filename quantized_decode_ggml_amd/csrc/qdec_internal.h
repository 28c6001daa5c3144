// Internal declarations shared by the libqdec translation units (host and
// device).  Not installed; the public ABI is include/qdec.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

namespace qdec {

// ---------------------------------------------------------------- layouts --
//
// Repacked Q8_0 matrix (one device allocation, 256-byte aligned planes):
//   q plane : n_out rows x n_in int8, row stride n_in bytes.  Row i's chunk c
//             (16 bytes, weights 16c..16c+15) is one aligned 16-byte load.
//   d plane : n_out rows x (n_in/32) fp16 scale bits, row stride n_in/32.
//   dT plane: the same scales block-major (n_in/32 rows of n_out), so that one
//             load gives a batched-GEMM tile the scales of many rows.
// Total bytes = n_out*n_in*18/16 (the GGML size plus the second scale plane)
// plus plane alignment; the GEMV kernels read the q and d planes only.
//
// Repacked Q4_K matrix:
//   qs plane : n_out rows x n_in/2 bytes of nibbles, in GGML order within each
//              super-block (128 bytes per super-block).
//   dm plane : n_out rows x (n_in/256) words, d | dmin << 16 (fp16 bits).
//   sm plane : n_out rows x (n_in/256) x 4 words; word p holds the unpacked
//              6-bit scales and mins of sub-blocks 2p and 2p+1:
//              sc[2p] | sc[2p+1] << 8 | m[2p] << 16 | m[2p+1] << 24.
//   (148 bytes per 256 weights instead of 144: the scales are unpacked once
//   here so the GEMV does not decode the 6-bit packing per lane.)
struct Q8View {
    const int8_t* q;
    const uint16_t* d;
    const uint16_t* dT;   // the scales again, block-major: dT[b * n_out + row] (batched GEMM)
};

// Fragment-tiled Q8_0 matrix (the matrix-core GEMV's copy): rows in groups of
// 16, the last group padded with zero rows; for group G and Q8_0 block b the
// 512-byte q tile at byte (G*nb + b)*512 holds, at byte 8*l, the 8 weights
// of row 16G + l%16 at k = 32b + 8*(l/16) .. +7 (the bf16 MFMA B-operand order
// of lane l), and the d plane holds at element (G*nb + b)*16 + r the scale of
// row 16G + r.  One wave load of a tile is 512 contiguous bytes.
struct Q8TView {
    const int8_t* q;
    const uint16_t* d;
};

struct Q4KView {
    const uint8_t* qs;
    const uint32_t* dm;
    const uint32_t* sm;
};

// Q6_K copy (256-weight super-blocks; GGML block: ql[128] low nibbles,
// qh[64] high bit pairs, int8 scales[16], fp16 d):
//   q plane : per super-block 16 chunks of 12 bytes; chunk 8h + m holds the
//             three GGML words ql[64h + 4m ..+3], ql[64h + 32 + 4m ..+3] and
//             qh[32h + 4m ..+3], i.e. the bits of the 16 weights
//             128h + 32j + 4m + t (j, t = 0..3); 192 bytes per super-block.
//   h plane : per super-block two 12-byte half headers: scales[8h ..8h+7],
//             fp16 d, two zero bytes.
//   (216 bytes per 256 weights instead of 210: one lane's 16 weights are one
//   contiguous 12-byte load and its scales and d one 12-byte load.)
struct Q6KView {
    const uint8_t* q;
    const uint8_t* h;
};

constexpr int64_t kAlign = 256;

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

inline int64_t q8_plane_bytes(int64_t n_in, int64_t n_out)
{
    return align_up(n_out * n_in, kAlign) + 2 * align_up(n_out * (n_in / 32) * 2, kAlign);
}

inline Q8View q8_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t off_d = align_up(n_out * n_in, kAlign);
    const int64_t off_dt = off_d + align_up(n_out * (n_in / 32) * 2, kAlign);
    return Q8View{reinterpret_cast<const int8_t*>(p), reinterpret_cast<const uint16_t*>(p + off_d),
                  reinterpret_cast<const uint16_t*>(p + off_dt)};
}

inline int64_t q8t_groups(int64_t n_out) { return (n_out + 15) / 16; }

inline int64_t q8t_plane_bytes(int64_t n_in, int64_t n_out)
{
    const int64_t tiles = q8t_groups(n_out) * (n_in / 32);
    return align_up(tiles * 512, kAlign) + align_up(tiles * 32, kAlign);
}

inline Q8TView q8t_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t tiles = q8t_groups(n_out) * (n_in / 32);
    return Q8TView{reinterpret_cast<const int8_t*>(p),
                   reinterpret_cast<const uint16_t*>(p + align_up(tiles * 512, kAlign))};
}

inline int64_t q6k_plane_bytes(int64_t n_in, int64_t n_out)
{
    const int64_t nsb = n_out * (n_in / 256);
    return align_up(nsb * 192, kAlign) + align_up(nsb * 24, kAlign);
}

inline Q6KView q6k_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t nsb = n_out * (n_in / 256);
    return Q6KView{reinterpret_cast<const uint8_t*>(p), reinterpret_cast<const uint8_t*>(p + align_up(nsb * 192, kAlign))};
}

// Cache type of the tiled copy (internal; the public types are the GGML ids).
constexpr int kTypeQ8_0Tiled = 0x108;

// Fragment-tiled Q4_K matrix (the one-row matrix-core GEMV's copy): rows in
// groups of 16 (the last padded with zero rows), 64-weight chunks c (chunk c
// = nibble bytes 32(c%4)..+31 of super-block c/4: low nibbles sub-block 2c,
// high nibbles 2c+1 of the row).  For group G:
//   q  : 512-byte tile (G*nch + c), lane l's 8 bytes at 8l = row 16G + l%16,
//        nibble bytes 32(c%4) + 8(l/16) .. +7 of super-block c/4;
//   sm : 64-byte tile (G*nch + c), word r = sc[2p] | sc[2p+1] << 8 | m[2p] << 16
//        | m[2p+1] << 24 of row 16G + r, p = c%4 (the 6-bit values unpacked);
//   dm : 64-byte tile (G*nsb + sb), word r = d | dmin << 16 (fp16 bits).
// 148 bytes per 256 weights, as the row-major Q4_K copy.
constexpr int kTypeQ4KTiled = 0x10C;

struct Q4KTView {
    const uint8_t* q;
    const uint32_t* sm;
    const uint32_t* dm;
};

__host__ __device__ inline int64_t q4kt_groups(int64_t n_out) { return (n_out + 15) / 16; }

inline int64_t q4kt_plane_bytes(int64_t n_in, int64_t n_out)
{
    const int64_t g = q4kt_groups(n_out), nch = n_in / 64, nsb = n_in / 256;
    return align_up(g * nch * 512, kAlign) + align_up(g * nch * 64, kAlign) + align_up(g * nsb * 64, kAlign);
}

inline Q4KTView q4kt_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t g = q4kt_groups(n_out), nch = n_in / 64;
    const int64_t off_sm = align_up(g * nch * 512, kAlign);
    const int64_t off_dm = off_sm + align_up(g * nch * 64, kAlign);
    return Q4KTView{reinterpret_cast<const uint8_t*>(p), reinterpret_cast<const uint32_t*>(p + off_sm),
                    reinterpret_cast<const uint32_t*>(p + off_dm)};
}

// Fragment-tiled Q6_K matrix (the one-row matrix-core GEMV's copy): rows in
// groups of 16 (the last padded with zero rows), 64-weight chunks c (chunk c
// = weights 64(c%4) .. +63 of super-block c/4: four 16-weight scale groups).
// For group G:
//   q  : 768-byte tile (G*nch + c), lane l's 12 bytes at 12l hold the 16
//        weights w_b = 64(c%4) + 16(l/16) + b (b = 0..15) of row 16G + l%16
//        as three words N0, N1, H: byte i of N0 is nib(w_i) | nib(w_4+i) << 4,
//        of N1 nib(w_8+i) | nib(w_12+i) << 4, and byte i of H carries
//        hi(w_4t+i) ^ 2 in bits 2t, 2t+1 (t = 0..3; nib and hi the low four
//        and high two bits of the 6-bit quant);
//   sc : 256-byte tile (G*nsb + sb), lane l's word at 4l: byte k is the
//        scale of group 4k + l/16 of row 16G + l%16 (chunk 4sb + k);
//   d  : 32-byte tile (G*nsb + sb), halfword r = d of row 16G + r (fp16 bits).
// 210 bytes per 256 weights, as the GGML block.
constexpr int kTypeQ6KTiled = 0x10E;

struct Q6KTView {
    const uint8_t* q;
    const uint32_t* sc;
    const uint16_t* d;
};

__host__ __device__ inline int64_t q6kt_groups(int64_t n_out) { return (n_out + 15) / 16; }

inline int64_t q6kt_plane_bytes(int64_t n_in, int64_t n_out)
{
    const int64_t g = q6kt_groups(n_out), nch = n_in / 64, nsb = n_in / 256;
    return align_up(g * nch * 768, kAlign) + align_up(g * nsb * 256, kAlign) + align_up(g * nsb * 32, kAlign);
}

inline Q6KTView q6kt_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t g = q6kt_groups(n_out), nch = n_in / 64, nsb = n_in / 256;
    const int64_t off_sc = align_up(g * nch * 768, kAlign);
    const int64_t off_d = off_sc + align_up(g * nsb * 256, kAlign);
    return Q6KTView{reinterpret_cast<const uint8_t*>(p), reinterpret_cast<const uint32_t*>(p + off_sc),
                    reinterpret_cast<const uint16_t*>(p + off_d)};
}

inline int64_t q4k_plane_bytes(int64_t n_in, int64_t n_out)
{
    const int64_t nsb = n_out * (n_in / 256);
    return align_up(n_out * (n_in / 2), kAlign) + align_up(nsb * 4, kAlign) + align_up(nsb * 16, kAlign);
}

inline Q4KView q4k_view(const void* base, int64_t n_in, int64_t n_out)
{
    const char* p = static_cast<const char*>(base);
    const int64_t nsb = n_out * (n_in / 256);
    const int64_t off_dm = align_up(n_out * (n_in / 2), kAlign);
    const int64_t off_sm = off_dm + align_up(nsb * 4, kAlign);
    return Q4KView{reinterpret_cast<const uint8_t*>(p), reinterpret_cast<const uint32_t*>(p + off_dm),
                   reinterpret_cast<const uint32_t*>(p + off_sm)};
}

// ------------------------------------------------------------- launchers --
// Each returns the hipError_t of its launch (hipGetLastError after launch).
// Arguments are validated by the caller (api.hip).

hipError_t launch_repack_q8_0(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                              hipStream_t s);
hipError_t launch_repack_q4k(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                             hipStream_t s);
hipError_t launch_repack_q8_0_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst,
                                    hipStream_t s);
hipError_t launch_repack_q6k(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s);
hipError_t launch_repack_q4k_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s);
hipError_t launch_repack_q6k_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s);
hipError_t launch_dequant_q6k(Q6KView w, int64_t n_in, int64_t n_out, float* out, hipStream_t s);
hipError_t launch_q6k_gemv(Q6KView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                           hipStream_t s);
hipError_t launch_dequant_q8_0(Q8View w, int64_t n_in, int64_t n_out, float* out, hipStream_t s);
hipError_t launch_dequant_q4k(Q4KView w, int64_t n_in, int64_t n_out, float* out, hipStream_t s);

enum GemvMode { kPlain = 0, kResidual = 1, kQKV = 2, kSwiGLU = 3 };

// Up to three row segments share one launch (QKV); SwiGLU uses segment 0 as
// gate and segment 1 as up, with the same rows.
struct Q8GemvProblem {
    GemvMode mode;
    int nseg;
    Q8View w[3];
    int64_t rows[3];
    float* out[3];
    const float* x;
    const float* residual;
    int64_t n_in;
    int64_t batch;
    // Optional RMSNorm of x folded into the product (one batch row on the
    // fast path only, see q8_gemv_norm_fusable): the kernel computes
    // r * sum_j W_ij (norm_w_j x_j), r = 1 / sqrt(mean_j x_j^2 + eps).
    const float* norm_w;
    float eps;
};

hipError_t launch_q8_0_gemv(const Q8GemvProblem& p, hipStream_t s);
bool q8_gemv_norm_fusable(const Q8GemvProblem& p);

// RMSNorm of `batch` rows of n floats: out = x / sqrt(mean(x^2) + eps) * w
// (one workgroup per row; out may be x).
hipError_t launch_rmsnorm(const float* x, int64_t n, int64_t batch, const float* w, float eps, float* out,
                          hipStream_t s);

// Matrix-core path for 3..8 batch rows (gemv_q8_0_mfma.hip).  It reads the
// fragment-tiled copies of the segments; where it splits K over workgroups
// it needs a device workspace of q8_mfma_workspace_bytes(mode, n_in, flat
// rows, batch) bytes for the slices' sums (0: none), owned by the caller and
// used in stream order.  Flat rows: the sum of the QKV segments, else the
// rows of the first matrix.
int64_t q8_mfma_workspace_bytes(int mode, int64_t n_in, int64_t rows, int64_t batch);
// Host-side extent check of the plan launch_q8_0_gemv_mfma would run with a
// workspace of ws_bytes: "" when every access stays inside its buffer, else
// a description of the overrun (the launcher refuses such a plan).
std::string q8_mfma_plan_check(const Q8GemvProblem& p, int64_t ws_bytes);
bool q8_mfma_supported(const Q8GemvProblem& p);
hipError_t launch_q8_0_gemv_mfma(const Q8GemvProblem& p, const Q8TView* tiles, void* workspace,
                                 hipStream_t s);

hipError_t launch_q4k_gemv(Q4KView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                           float* out, hipStream_t s);
// One batch row on the integer matrix cores from the tiled copy (n_in one of
// 1024, 2048, 3072, 4096, 6144, 8192); q4k_mfma_supported says whether it
// takes the shape.
// 2..8 batch rows run the rows kernel on the same copy (whole rows up to 4096
// columns; 6144 and 8192 up to 4 rows).  q4k_mfma_plan_check: host-side
// extent check of either plan ("" when every access stays inside).
bool q4k_mfma_supported(int64_t n_in, int64_t batch);
std::string q4k_mfma_plan_check(int64_t n_in, int64_t n_out, int64_t batch);
hipError_t launch_q4k_gemv_mfma(Q4KTView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                                hipStream_t s);
// The same for Q6_K (n_in one of 1024, 2048, 3072, 4096, 6144, 8192; also
// 2..8 batch rows while the rows x width fit LDS), with a host-side extent
// check of its plan ("" when every access stays inside the tiled copy, x and
// out; the launcher refuses any other plan).
bool q6k_mfma_supported(int64_t n_in, int64_t batch);
std::string q6k_mfma_plan_check(int64_t n_in, int64_t n_out, int64_t batch);
hipError_t launch_q6k_gemv_mfma(Q6KTView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                                hipStream_t s);

// Batched GEMM over a Q8_0 copy.  With a workspace of q8_gemm_workspace_bytes,
// on shapes the pipelined kernel takes x is first rounded to bf16 there and the
// DMA-fed kernel runs; on the others the register-staged kernel keeps the
// partial products of its K slices there and a small kernel sums them in slice
// order.  Without a workspace the register-staged kernel runs and adds its K
// slices with f32 atomics into a zeroed output (same products, summation order
// not fixed).
int64_t q8_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch);
hipError_t launch_q8_0_gemm(Q8View w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                            float* out, void* workspace, hipStream_t s);
// Dense f32 weights.  With the weight's bf16 copy (wbf16, made by
// qdec_prepare), n_in % 64 == 0 and a workspace of f32_gemm_workspace_bytes(...,
// true), the DMA-fed kernel reads that copy (x rounded to bf16 and the K-slice
// partials in the workspace); else the register-staged kernel rounds W as it
// loads it, with the K-slice partials in a workspace of
// f32_gemm_workspace_bytes(..., false) when there is one, as above.  Both
// contract bf16(W) with bf16(x) in f32.
int64_t f32_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch, bool bf16_copy);
// Host-side extent checks of the batched-GEMM plans (DMA-fed kernel for Q8_0
// weights or a bf16 copy, register-staged kernel otherwise) with a workspace
// of ws_bytes (0: none); "" when every access stays inside its buffer.
std::string q8_gemm_plan_check(int64_t n_in, int64_t n_out, int64_t batch, int64_t ws_bytes);
std::string f32_gemm_plan_check(int64_t n_in, int64_t n_out, int64_t batch, bool bf16_copy, int64_t ws_bytes);
hipError_t launch_f32_gemm(const float* w, const void* wbf16, int64_t n_in, int64_t n_out, int64_t batch,
                           const float* x, float* out, void* workspace, hipStream_t s);
// dst[i] = bf16(src[i]) (round to nearest even), count % 4 == 0: the bf16 copy
// of a dense f32 weight.
hipError_t launch_to_bf16(const float* src, int64_t count, void* dst, hipStream_t s);

// Top-k of batch rows of n_out logits (1 <= k <= 256).  The workspace holds
// the candidate lists: batch * chunks * k 64-bit keys for the two-launch
// select, two buffers for the staged path it falls back to past its merge
// capacity (none there for a single chunk).
int64_t topk_workspace_bytes(int64_t n_out, int64_t batch, int k);
hipError_t launch_topk(const float* logits, int64_t n_out, int64_t batch, int k, void* workspace,
                       int32_t* top_idx, float* top_val, hipStream_t s);

// Decode attention (attention.hip): RoPE + KV append, and GQA attention over
// n_ctx cached positions (head_dim 64 or 128, <= 16 query heads per kv head;
// the workspace holds per-chunk partials, none for n_ctx <= 128).
int64_t attention_workspace_bytes(int64_t n_head, int64_t head_dim, int64_t n_ctx);
hipError_t launch_rope_append(float* q, float* k, const float* v, int64_t n_head, int64_t n_kv, int64_t d, int64_t pos,
                              double base, float* k_cache, float* v_cache, int64_t max_seq, hipStream_t s);
hipError_t launch_attention(const float* q, const float* k_cache, const float* v_cache, int64_t n_head, int64_t n_kv,
                            int64_t d, int64_t n_ctx, int64_t max_seq, float scale, float* out, void* workspace,
                            hipStream_t s);

hipError_t launch_empty(hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);
// loads_per_lane in {1, 2, 4, 8, 16}; bytes % 16 == 0
hipError_t launch_stream_read(const void* src, int64_t bytes, int loads_per_lane, uint32_t* sink, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

// Kernel-launch counter (a witness that the device path ran).
void count_launch(uint64_t n = 1);

}  // namespace qdec
