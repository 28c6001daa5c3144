// Q4_K dequant-GEMV for gfx950 (rustdoc "Module cuda_lane", Functions
// section: try_q4k_soa_gemv, on-device Q4_K dequant-GEMV over a repacked
// layout), batch 1..8.
//
// Super-block (256 weights, 144 bytes; the Q4_K workload definition that
// accompanies the pages): fp16 d, fp16 dmin, 12 bytes of eight 6-bit scales
// and mins (GGML K-quant packing), 128 nibble bytes.  In 64-element chunk p the
// low nibbles of qs[32p..32p+31] are sub-block 2p and the high nibbles
// sub-block 2p+1.  w = d*sc*q - dmin*m.
//
// Work mapping: as the Q8_0 kernel, with a 16-byte chunk of nibbles per lane
// (32 weights: 16 of sub-block 2p and 16 of sub-block 2p+1).  Per chunk the
// dot product is taken per sub-block in the factored form
//     sum_t w_t x_t = (d*sc) * sum_t q_t x_t - (dmin*m) * sum_t x_t,
// where both products d*sc and dmin*m are exact in f32.  sum_t x_t depends only
// on the lane's columns, so it is computed once per chunk and reused for the R
// rows of the tile.
#include "qdec_internal.h"

namespace qdec {

namespace {

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

__device__ inline uint32_t scale_byte(const uint4& m, int idx)
{
    const uint32_t word = idx < 4 ? m.y : (idx < 8 ? m.z : m.w);
    return (word >> (8 * (idx & 3))) & 0xffu;
}

// 6-bit scale and min of sub-block s (GGML K-quant packing): sub-blocks 0-3
// use the low 6 bits of scale bytes s and s+4; sub-blocks 4-7 take their low 4
// bits from byte s+4 (scale: low nibble, min: high nibble) and their high 2
// bits from the top of bytes s-4 (scale) and s (min).
__device__ inline void scale_min(const uint4& m, int s, float& sc, float& mn)
{
    uint32_t a, b;
    if (s < 4) {
        a = scale_byte(m, s) & 63u;
        b = scale_byte(m, s + 4) & 63u;
    } else {
        const uint32_t lo = scale_byte(m, s + 4);
        a = (lo & 15u) | ((scale_byte(m, s - 4) >> 6) << 4);
        b = (lo >> 4) | ((scale_byte(m, s) >> 6) << 4);
    }
    sc = (float)a;
    mn = (float)b;
}

struct Q4KArgs {
    const uint8_t* qs;
    const uint4* meta;
    float* out;
    const float* x;
    int64_t n_in;
    int64_t n_out;
    int batch;
    int lpr_log2;
    int nch;  // 16-byte nibble chunks per row = n_in / 32
};

template <int B, int R, int NCH>
__global__ __launch_bounds__(256) void q4k_gemv_kernel(Q4KArgs a)
{
    const int lpr = 1 << a.lpr_log2;
    const int lane = threadIdx.x & 63;
    const int g = lane >> a.lpr_log2;
    const int j = lane & (lpr - 1);
    const int groups = 64 >> a.lpr_log2;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t row0 = wave * groups * R;
    const int64_t nsb = a.n_in >> 8;

    const uint8_t* qrow[R];
    const uint4* mrow[R];
    int64_t rowid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + (int64_t)r * groups + g;
        rowid[r] = row;
        const int64_t rr = row < a.n_out ? row : a.n_out - 1;
        qrow[r] = a.qs + rr * (a.n_in >> 1);
        mrow[r] = a.meta + rr * nsb;
    }
    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;

    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

    const int nk = NCH > 0 ? NCH : (a.nch + lpr - 1) >> a.lpr_log2;
#pragma unroll
    for (int kc = 0; kc < (NCH > 0 ? NCH : 1); ++kc) {
        for (int kk = 0; kk < (NCH > 0 ? 1 : nk); ++kk) {
            const int c = j + ((NCH > 0 ? kc : kk) << a.lpr_log2);
            if (NCH == 0 && c >= a.nch) break;
            const int sb = c >> 3;
            const int cc = c & 7;
            const int p = cc >> 1, h = cc & 1;
            uint4 qv[R], mv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                qv[r] = *reinterpret_cast<const uint4*>(qrow[r] + (int64_t)c * 16);
                mv[r] = mrow[r][sb];
            }
            // per-row sub-block factors (independent of the batch row)
            float f_lo[R], g_lo[R], f_hi[R], g_hi[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float d = fp16_bits_to_f32((uint16_t)(mv[r].x & 0xffff));
                const float dmin = fp16_bits_to_f32((uint16_t)(mv[r].x >> 16));
                float sc, mn;
                scale_min(mv[r], 2 * p, sc, mn);
                f_lo[r] = d * sc;
                g_lo[r] = dmin * mn;
                scale_min(mv[r], 2 * p + 1, sc, mn);
                f_hi[r] = d * sc;
                g_hi[r] = dmin * mn;
            }
            const int64_t xoff = (int64_t)sb * 256 + 64 * p + 16 * h;
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float xl[16], xh[16];
                const float4* pl = reinterpret_cast<const float4*>(xrow[b] + xoff);
                const float4* ph = reinterpret_cast<const float4*>(xrow[b] + xoff + 32);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float4 v = pl[k], u = ph[k];
                    xl[4 * k] = v.x; xl[4 * k + 1] = v.y; xl[4 * k + 2] = v.z; xl[4 * k + 3] = v.w;
                    xh[4 * k] = u.x; xh[4 * k + 1] = u.y; xh[4 * k + 2] = u.z; xh[4 * k + 3] = u.w;
                }
                float sl = xl[0], sh = xh[0];
#pragma unroll
                for (int t = 1; t < 16; ++t) {
                    sl += xl[t];
                    sh += xh[t];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t w4[4] = {qv[r].x, qv[r].y, qv[r].z, qv[r].w};
                    float tl = 0.0f, th = 0.0f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t lo = w4[k] & 0x0f0f0f0fu;
                        const uint32_t hi = (w4[k] >> 4) & 0x0f0f0f0fu;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            tl = __builtin_fmaf((float)((lo >> (8 * t)) & 0xffu), xl[4 * k + t], tl);
                            th = __builtin_fmaf((float)((hi >> (8 * t)) & 0xffu), xh[4 * k + t], th);
                        }
                    }
                    float v = acc[r][b];
                    v = __builtin_fmaf(f_lo[r], tl, v);
                    v = __builtin_fmaf(-g_lo[r], sl, v);
                    v = __builtin_fmaf(f_hi[r], th, v);
                    v = __builtin_fmaf(-g_hi[r], sh, v);
                    acc[r][b] = v;
                }
            }
        }
    }

    for (int off = lpr >> 1; off > 0; off >>= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] += __shfl_xor(acc[r][b], off);
    }
    if (j != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (rowid[r] >= a.n_out) continue;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (b >= a.batch) break;
            a.out[(int64_t)b * a.n_out + rowid[r]] = acc[r][b];
        }
    }
}

using KernelFn = void (*)(Q4KArgs);

template <int B, int R>
KernelFn pick_nch(int n)
{
    switch (n) {
        case 1: return q4k_gemv_kernel<B, R, 1>;
        case 2: return q4k_gemv_kernel<B, R, 2>;
        case 3: return q4k_gemv_kernel<B, R, 3>;
        case 4: return q4k_gemv_kernel<B, R, 4>;
        default: return q4k_gemv_kernel<B, R, 0>;
    }
}

}  // namespace

hipError_t launch_q4k_gemv(Q4KView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                           float* out, hipStream_t s)
{
    Q4KArgs a{};
    a.qs = w.qs;
    a.meta = w.meta;
    a.out = out;
    a.x = x;
    a.n_in = n_in;
    a.n_out = n_out;
    a.batch = (int)batch;
    a.nch = (int)(n_in / 32);
    // Largest power-of-two lane count (<= 64) that divides the chunk count, so
    // that row groups cover whole rows without a ragged tail when possible.
    int lpr_log2 = 6;
    while (lpr_log2 > 3 && (a.nch % (1 << lpr_log2)) != 0) --lpr_log2;
    if (a.nch % (1 << lpr_log2) != 0) lpr_log2 = 6;
    int nch_per_lane = a.nch % (1 << lpr_log2) == 0 ? a.nch >> lpr_log2 : 0;
    if (nch_per_lane > 4) nch_per_lane = 0;
    a.lpr_log2 = lpr_log2;
    const int groups = 64 >> lpr_log2;

    const int bt = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
    int r = 4;
    while (r > 1 && n_out / ((int64_t)groups * r) < 1024 * (r == 4 ? 2 : 1)) r >>= 1;
    KernelFn fn;
    int r_eff = r;
    switch (bt) {
        case 1: fn = r == 4 ? pick_nch<1, 4>(nch_per_lane) : r == 2 ? pick_nch<1, 2>(nch_per_lane)
                                                                   : pick_nch<1, 1>(nch_per_lane);
            break;
        case 2: fn = r >= 2 ? pick_nch<2, 2>(nch_per_lane) : pick_nch<2, 1>(nch_per_lane);
            r_eff = r >= 2 ? 2 : 1;
            break;
        case 4: fn = r >= 2 ? pick_nch<4, 2>(nch_per_lane) : pick_nch<4, 1>(nch_per_lane);
            r_eff = r >= 2 ? 2 : 1;
            break;
        default: fn = pick_nch<8, 1>(nch_per_lane); r_eff = 1; break;
    }
    const int64_t rows_per_wave = (int64_t)groups * r_eff;
    const int64_t waves = (n_out + rows_per_wave - 1) / rows_per_wave;
    hipLaunchKernelGGL(fn, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
