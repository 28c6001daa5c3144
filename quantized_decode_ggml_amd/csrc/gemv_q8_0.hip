// Q8_0 dequant-GEMV family for gfx950: plain, residual epilogue, fused QKV
// (GQA) and fused SwiGLU, batch 1..8.
//
// What is computed (rustdoc "Module cuda_lane", Functions section):
//   try_q8_0_cuda_gemv / q8_0_gemv_oracle_into : out[b][i] = sum_j (d*q)[i][j] x[b][j]
//   try_q4k_soa_ffn_block_residual             : out = residual + W x
//   try_q4k_soa_qkv                            : q, k, v from one shared x;
//                                                K and V have n_kv rows
//   try_q4k_soa_fused_swiglu                   : out[i] = silu(gate_i.x) * (up_i.x)
//
// The weights are read exactly once, so every variant is bound by HBM; the
// design keeps the whole weight stream of a workgroup in flight from its first
// instructions and finishes each output row inside one workgroup (device-wide
// reductions would need cross-XCD fences, which cost more than the kernel).
//
// Fast path (n_in a multiple of 1024, chunks per row NCH = n_in/1024 in
// {1,2,3,4,6,8,12,16}): a row's 16-byte chunks are split over the 64 lanes of a
// wave (lane j takes chunks j, j+64, ...) and over KS waves of the workgroup
// (each takes CH = NCH/KS consecutive chunk columns).  A wave computes R rows
// (x 2 matrices for SwiGLU) at once, so each x value in registers serves R
// rows.  Per wave the order is: x of its columns (registers), every fp16 scale,
// every q chunk, then the arithmetic, so the loads return in use order while
// later ones are still in flight.  One batch row: x is copied once per
// workgroup into LDS (direct global->LDS loads issued before the weight
// loads) and shared by several row groups, and a wave takes one or two rows
// whole or split over few waves; with a folded RMSNorm x stays in registers,
// one chunk column per wave and one row group per workgroup, which keeps the
// arithmetic a wave still owes after its last load short (the kernel's tail).
// A residual is fetched by the storing lanes before the weight stream.  The scalar set-up
// before the first weight load is kept to a few dozen instructions: the
// scalar unit is shared by every wave of a compute unit, and all of them
// start together.  With several batch rows whose x does not
// fit in registers, the workgroup first copies x into LDS (direct
// global->LDS loads, before the weight loads) when it fits in 48 KB; wider
// cases read x from L2 chunk by chunk.  Lane sums are folded with DPP row
// operations and lane reads into scalar registers (no LDS), the KS wave
// partials through LDS.
//
// General path (other n_in): rows are split over "row groups" of LPR lanes
// (LPR = largest power of two not above the chunk count), with a bounds-checked
// chunk loop and shuffle reductions.
//
// Arithmetic per chunk: t = sum of 16 products q*x (f32 FMA chain), then
// acc = fma(d, t, acc), then the lane tree.  The longest rounding chain is
// 16 + NCH + 6 + 2 operations (32 at n_in = 8192), so
// |err| <= 33 * 2^-24 * sum_j|w x| < 2e-6 * sum_j|w x|, inside the 1e-5 bound.
#include "gemv_common.h"

namespace qdec {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));




// Sum of 16 products of the int8 weights in `qv` with x[0..15].
__device__ inline float dot16(const uint4& qv, const float* x)
{
    const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
    float t = (float)(int8_t)(w[0] & 0xff) * x[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int b = (k == 0 ? 1 : 0); b < 4; ++b)
            t = __builtin_fmaf((float)(int8_t)((w[k] >> (8 * b)) & 0xff), x[4 * k + b], t);
    }
    return t;
}

// Weight bytes are read once per launch: non-temporal loads keep them from
// displacing x and the outputs in the caches.
__device__ inline uint4 stream_load16(const int8_t* p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint16_t stream_load2(const uint16_t* p) { return __builtin_nontemporal_load(p); }

__device__ inline void load_x16(const float* p, float (&xv)[16])
{
    const float4* xp = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 v = xp[k];
        xv[4 * k] = v.x; xv[4 * k + 1] = v.y; xv[4 * k + 2] = v.z; xv[4 * k + 3] = v.w;
    }
}

template <int CTRL>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wave, result in every lane: rotations and quad
// permutes within each 16-lane row (DPP), then the four row sums read into
// scalar registers.  (The gfx950 permlane swaps would need two distinct copies
// of the value; the compiler merges equal operands into one register.)
__device__ inline float wave_sum(float v)
{
    v += dpp<0x128>(v);  // row_ror:8
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// x staged in LDS (batch > 1): the batch x n_in activations are copied into
// LDS once per workgroup by direct global->LDS loads issued before any weight
// load, so they never queue behind the weight stream.  Layout: the flattened
// x as 16-float chunks c, the four float4 of chunk c stored in the order
// q ^ ((c >> 1) & 3), which spreads the 64-byte per-lane reads of eight
// neighbouring lanes over distinct LDS banks.
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline int xs_slot(int c, int q) { return 4 * c + (q ^ ((c >> 1) & 3)); }

__device__ inline void lds_x16(const float* xs, int c, float (&xv)[16])
{
    const float4* xp = reinterpret_cast<const float4*>(xs);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = xp[xs_slot(c, q)];
        xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
    }
}

template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt N (low 4 bits + high 2 bits); expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Fast path.  MODE: GemvMode.  B: batch rows handled (>= the real batch;
// padding rows use the last real x row and are never stored).  R: rows per
// wave.  CH: chunk columns per lane in this wave.  KS: waves per row group.
// XL: x staged in LDS (dynamic shared memory of batch * n_in floats).  NW:
// waves per workgroup (NW / KS row groups).
template <int MODE, int B, int R, int CH, int KS, bool XL, int NW>
__global__ __launch_bounds__(64 * NW) void q8_0_gemv_fast(Q8GemvArgs a)
{
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;   // weight matrices per output row
    constexpr int GROUPS = NW / KS;                  // row groups per workgroup
    static_assert(GROUPS * KS == NW, "whole row groups per workgroup");
    constexpr bool XREG = !XL && B * CH <= 4;        // x in registers (<= 64 VGPRs)
    __shared__ float part[KS > 1 ? NW : 1][R][NM][B];
    __shared__ double part_ss[KS > 1 && B == 1 ? NW : 1];    // folded RMSNorm: sum of squares per wave
    extern __shared__ __attribute__((aligned(16))) float xs[];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = w / KS, ks = w % KS;
    const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + grp) * R;
    const int cbase = ks * CH;                       // first chunk column of this wave

    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;

    if constexpr (XL) {
        // batch * n_in / 4 float4 slots, 64 per wave and step; slot s of the
        // layout holds global float4 4c + (j ^ ((c >> 1) & 3)), c = s / 4
        const int nslot = (int)(((int64_t)a.batch * a.n_in) >> 2);
        for (int sb = w * 64; sb < nslot; sb += 64 * NW) {
            const int c = (sb + lane) >> 2, j = (sb + lane) & 3;
            const float* src = a.x + (int64_t)(4 * c + (j ^ ((c >> 1) & 3))) * 4;
            if (sb + lane < nslot) __builtin_amdgcn_global_load_lds(src, (lds_void*)(xs + sb * 4), 16, 0, 0);
        }
        // the vmcnt wait below counts only the weight loads issued after these
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    float xr[XREG ? CH : 1][XREG ? B : 1][16];
    if constexpr (XREG) {
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
            for (int b = 0; b < B; ++b) load_x16(xrow[b] + (int64_t)(lane + 64 * (cbase + k)) * 16, xr[k][b]);
    }
    // Residual epilogue: the storing lanes fetch their residual value before
    // the weight stream, so no load round trip is left for the kernel's tail.
    float rpre = 0.0f;
    if constexpr (MODE == kResidual) {
        const int rl = lane / B, bl = lane % B;
        if (ks == 0 && lane < R * B && bl < a.batch && row0 + rl < a.total_rows)
            rpre = a.residual[(int64_t)bl * a.total_rows + row0 + rl];
    }
    // One batch row may fold an RMSNorm of x into the product: the norm
    // weights of the wave's columns are loaded with x (before the weight
    // stream) and applied after the weight loads are issued.
    constexpr bool NORM_OK = B == 1 && XREG;
    const bool norm = NORM_OK && a.norm_w != nullptr;
    float gr[NORM_OK ? CH : 1][16];
    if constexpr (NORM_OK) {
        if (norm) {
#pragma unroll
            for (int k = 0; k < CH; ++k) load_x16(a.norm_w + (int64_t)(lane + 64 * (cbase + k)) * 16, gr[k]);
        }
    }

    // Row pointers (scalar work shared by every wave of a CU, so kept short):
    // when the R rows are all in range and in one segment they are consecutive
    // rows of one plane; otherwise each row is mapped (and clamped) alone.
    Seg sg[R][NM];
    if (row0 + R <= a.total_rows && same_segment<MODE>(a, row0, row0 + R - 1)) {
        const int64_t nb = a.n_in >> 5;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const Seg s0 = row_seg<MODE>(a, row0, m);
#pragma unroll
            for (int r = 0; r < R; ++r) sg[r][m] = Seg{s0.q + r * a.n_in, s0.d + r * nb};
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rw = row0 + r;
            const int64_t rr = rw < a.total_rows ? rw : a.total_rows - 1;  // keep loads in bounds
#pragma unroll
            for (int m = 0; m < NM; ++m) sg[r][m] = row_seg<MODE>(a, rr, m);
        }
    }
    uint16_t dv[CH][R][NM];
    uint4 qv[CH][R][NM];
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < NM; ++m) dv[k][r][m] = stream_load2(sg[r][m].d + ((lane + 64 * (cbase + k)) >> 1));
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < NM; ++m)
                qv[k][r][m] = stream_load16(sg[r][m].q + (int64_t)(lane + 64 * (cbase + k)) * 16);
    // The weight loads must stay ahead of the arithmetic (the weight planes
    // are not marked restrict, so this fence pins them).
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XL) {
        // this wave's x slots have landed once at most the weight loads remain;
        // the barrier makes every wave's slots visible
        wait_vmcnt<2 * CH * R * NM>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    // folded RMSNorm: x <- norm_w * x, and this lane's share of sum x^2 (f64:
    // no overflow for any f32 row, and the sum is exact to f64 rounding)
    double ssq = 0.0;
    if constexpr (NORM_OK) {
        if (norm) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const float v = xr[k][0][t];
                    ssq = __builtin_fma((double)v, (double)v, ssq);
                    xr[k][0][t] = v * gr[k][t];
                }
        }
    }

    float acc[R][NM][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][m][b] = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        if constexpr (B == 1) {
            // one batch row: convert and multiply in one pass
            float xv[16];
            if constexpr (XREG) {
#pragma unroll
                for (int t = 0; t < 16; ++t) xv[t] = xr[XREG ? k : 0][0][t];
            } else if constexpr (XL) {
                lds_x16(xs, lane + 64 * (cbase + k), xv);
            } else {
                load_x16(xrow[0] + (int64_t)(lane + 64 * (cbase + k)) * 16, xv);
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc[r][m][0] = __builtin_fmaf(fp16_bits_to_f32(dv[k][r][m]), dot16(qv[k][r][m], xv),
                                                  acc[r][m][0]);
        } else {
            // several batch rows: convert each weight once, then B dot products
            float qf[R][NM][16];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const uint32_t wd[4] = {qv[k][r][m].x, qv[k][r][m].y, qv[k][r][m].z, qv[k][r][m].w};
#pragma unroll
                    for (int t = 0; t < 16; ++t) qf[r][m][t] = (float)(int8_t)((wd[t >> 2] >> (8 * (t & 3))) & 0xff);
                }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float xv[16];
                if constexpr (XREG) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) xv[t] = xr[XREG ? k : 0][XREG ? b : 0][t];
                } else if constexpr (XL) {
                    const int bb = b < a.batch ? b : a.batch - 1;
                    lds_x16(xs, bb * (int)(a.n_in >> 4) + lane + 64 * (cbase + k), xv);
                } else {
                    load_x16(xrow[b] + (int64_t)(lane + 64 * (cbase + k)) * 16, xv);
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        float t = qf[r][m][0] * xv[0];
#pragma unroll
                        for (int i = 1; i < 16; ++i) t = __builtin_fmaf(qf[r][m][i], xv[i], t);
                        acc[r][m][b] = __builtin_fmaf(fp16_bits_to_f32(dv[k][r][m]), t, acc[r][m][b]);
                    }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][m][b] = wave_sum(acc[r][m][b]);

    if constexpr (NORM_OK) {
        if (norm) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ssq += __shfl_xor(ssq, off);
        }
    }
    // lane l < R*B ends up with the (row l / B, batch row l % B) value
    float v0 = 0.0f, v1 = 0.0f;
    if constexpr (KS > 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int b = 0; b < B; ++b) part[w][r][m][b] = acc[r][m][b];
            if constexpr (NORM_OK) part_ss[w] = ssq;
        }
        __syncthreads();
        if (ks != 0) return;
        if (lane < R * B) {
            const int r = lane / B, b = lane % B;
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                v0 += part[w + k][r][0][b];
                v1 += part[w + k][r][NM - 1][b];
            }
        }
        if constexpr (NORM_OK) {
            if (norm) {
                double t = 0.0;
#pragma unroll
                for (int k = 0; k < KS; ++k) t += part_ss[w + k];
                ssq = t;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                if (lane == r * B + b) {
                    v0 = acc[r][0][b];
                    v1 = acc[r][NM - 1][b];
                }
    }
    if constexpr (NORM_OK) {
        if (norm) {
            const float rs = (float)(1.0 / sqrt(ssq / (double)a.n_in + (double)a.eps));
            v0 *= rs;
            v1 *= rs;
        }
    }
    const int rl = lane / B, bl = lane % B;
    if (lane < R * B && bl < a.batch && row0 + rl < a.total_rows) {
        if constexpr (MODE == kResidual) a.out0[(int64_t)bl * a.total_rows + row0 + rl] = rpre + v0;
        else store_row<MODE>(a, row0 + rl, bl, v0, v1);
    }
}

// General path: row groups of LPR lanes, one row per group, bounds-checked loop.
template <int MODE, int B>
__global__ __launch_bounds__(256) void q8_0_gemv_general(Q8GemvArgs a)
{
    constexpr int NM = (MODE == kSwiGLU) ? 2 : 1;
    const int lpr = 1 << a.lpr_log2;
    const int lane = threadIdx.x & 63;
    const int g = lane >> a.lpr_log2;
    const int j = lane & (lpr - 1);
    const int groups = 64 >> a.lpr_log2;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);

    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;

    const int64_t row = wave * groups + g;
    const int64_t rr = row < a.total_rows ? row : a.total_rows - 1;
    Seg sg[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) sg[m] = row_seg<MODE>(a, rr, m);
    float acc[NM][B];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;
    for (int c = j; c < a.nch; c += lpr) {
        uint4 qv[NM];
        uint16_t dv[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            dv[m] = stream_load2(sg[m].d + (c >> 1));
            qv[m] = stream_load16(sg[m].q + (int64_t)c * 16);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float xv[16];
            load_x16(xrow[b] + (int64_t)c * 16, xv);
#pragma unroll
            for (int m = 0; m < NM; ++m)
                acc[m][b] = __builtin_fmaf(fp16_bits_to_f32(dv[m]), dot16(qv[m], xv), acc[m][b]);
        }
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[m][b] += __shfl_xor(acc[m][b], off);
    }
    if (j != 0 || row >= a.total_rows) return;
#pragma unroll
    for (int b = 0; b < B; ++b)
        if (b < a.batch) store_row<MODE>(a, row, b, acc[0][b], acc[NM - 1][b]);
}

using KernelFn = void (*)(Q8GemvArgs);

// Fast-path instantiations for two or more batch rows: (CH, KS) from the
// chunk count per row, four waves per workgroup; R from the row count; B from
// the batch.  Register use grows with R*NM*B, so wide batches and SwiGLU take
// fewer rows per wave.
template <int MODE, int B, int R, bool XL>
KernelFn pick_split(int nch64)
{
    switch (nch64) {
        case 1: return q8_0_gemv_fast<MODE, B, R, 1, 1, XL, 4>;
        case 2: return q8_0_gemv_fast<MODE, B, R, 2, 1, XL, 4>;
        case 3: return q8_0_gemv_fast<MODE, B, R, 3, 1, XL, 4>;
        case 4: return q8_0_gemv_fast<MODE, B, R, 2, 2, XL, 4>;
        case 6: return q8_0_gemv_fast<MODE, B, R, 3, 2, XL, 4>;
        case 8: return q8_0_gemv_fast<MODE, B, R, 2, 4, XL, 4>;
        case 12: return q8_0_gemv_fast<MODE, B, R, 3, 4, XL, 4>;
        case 16: return q8_0_gemv_fast<MODE, B, R, 4, 4, XL, 4>;
        default: return nullptr;
    }
}

int split_ks(int nch64) { return nch64 <= 3 ? 1 : (nch64 <= 6 ? 2 : 4); }

// R actually instantiated for (mode, requested r): SwiGLU streams two
// matrices per row, so it takes at most two rows.
int fast_r(GemvMode mode, int bt, int r)
{
    (void)bt;
    if (mode == kSwiGLU) return r >= 2 ? 2 : 1;
    return r;
}

template <int MODE, int B, bool XL>
KernelFn pick_rows(int r, int nch64)
{
    if constexpr (MODE == kSwiGLU) {
        return r >= 2 ? pick_split<MODE, B, 2, XL>(nch64) : pick_split<MODE, B, 1, XL>(nch64);
    } else {
        return r == 4 ? pick_split<MODE, B, 4, XL>(nch64)
                      : (r == 2 ? pick_split<MODE, B, 2, XL>(nch64) : pick_split<MODE, B, 1, XL>(nch64));
    }
}

template <int MODE>
KernelFn pick_fast(int bt, int r, int nch64, bool xl)
{
    switch (bt) {
        case 2: return xl ? pick_rows<MODE, 2, true>(r, nch64) : pick_rows<MODE, 2, false>(r, nch64);
        case 4: return xl ? pick_rows<MODE, 4, true>(r, nch64) : pick_rows<MODE, 4, false>(r, nch64);
        default: return xl ? pick_rows<MODE, 8, true>(r, nch64) : pick_rows<MODE, 8, false>(r, nch64);
    }
}

// One batch row.  A wave's arithmetic after its last weight load lands is the
// kernel's tail (a single wave issues a signed-byte conversion only every ~13
// cycles), so each wave takes one chunk column (two above 8192 columns) and a
// workgroup is the KS waves of one row group; x is then read once per
// workgroup.  Rows per wave: 8 weight rows up to four waves per group, 4
// beyond, halved while the grid would hold fewer than 3072 waves (three per
// SIMD).
struct B1Shape { int ks, ch; };

B1Shape b1_shape(int nch64)
{
    switch (nch64) {
        case 1: return {1, 1};
        case 2: return {2, 1};
        case 3: return {3, 1};
        case 4: return {4, 1};
        case 6: return {6, 1};
        case 8: return {8, 1};
        case 12: return {6, 2};
        case 16: return {8, 2};
        default: return {0, 0};
    }
}

int b1_rows(GemvMode mode, int ks, int64_t total_rows)
{
    const int nm = mode == kSwiGLU ? 2 : 1;
    int r = (ks <= 4 ? 8 : 4) / nm;
    while (r > 1 && (total_rows / r) * ks < 3072) r >>= 1;
    return r;
}

template <int MODE, int R>
KernelFn pick_b1_split(int nch64)
{
    switch (nch64) {
        case 1: return q8_0_gemv_fast<MODE, 1, R, 1, 1, false, 1>;
        case 2: return q8_0_gemv_fast<MODE, 1, R, 1, 2, false, 2>;
        case 3: return q8_0_gemv_fast<MODE, 1, R, 1, 3, false, 3>;
        case 4: return q8_0_gemv_fast<MODE, 1, R, 1, 4, false, 4>;
        case 6: return q8_0_gemv_fast<MODE, 1, R, 1, 6, false, 6>;
        case 8: return q8_0_gemv_fast<MODE, 1, R, 1, 8, false, 8>;
        case 12: return q8_0_gemv_fast<MODE, 1, R, 2, 6, false, 6>;
        case 16: return q8_0_gemv_fast<MODE, 1, R, 2, 8, false, 8>;
        default: return nullptr;
    }
}

template <int MODE>
KernelFn pick_b1(int r, int nch64)
{
    if constexpr (MODE == kSwiGLU) {
        return r >= 4 ? pick_b1_split<MODE, 4>(nch64)
                      : (r == 2 ? pick_b1_split<MODE, 2>(nch64) : pick_b1_split<MODE, 1>(nch64));
    } else {
        return r >= 8 ? pick_b1_split<MODE, 8>(nch64)
                      : (r == 4 ? pick_b1_split<MODE, 4>(nch64)
                                : (r == 2 ? pick_b1_split<MODE, 2>(nch64) : pick_b1_split<MODE, 1>(nch64)));
    }
}

// One batch row with x staged in LDS (no folded norm, one weight matrix per
// row): G row groups of a workgroup share one LDS copy of x, and a wave takes
// R whole rows (n_in <= 4096) or a row's K split over KS waves (wider rows).
// Measured against the register shapes (graph-replayed launches over rotated
// copies): fewer cross-wave reductions, and x read from L2 once per
// workgroup instead of once per wave.  Up to 4096 columns one row per wave,
// 8 row groups, 4 while that leaves fewer than 1024 workgroups (8192x3072:
// 6.6 -> 6.0-6.1 us; 5120x3072: 4.96 -> 4.75 us), and two rows per wave in 4
// groups for very tall matrices (128256x3072: 67 -> 62 us); 8192 columns two rows per
// wave, four waves per row, two groups (3072x8192 with residual: 7.0 ->
// 6.7-6.8 us).
struct B1XlShape { int ks, ch, g, r; };

B1XlShape b1_xl_shape(int nch64, int64_t total_rows)
{
    if (nch64 >= 1 && nch64 <= 4) {
        if (total_rows / 8 >= 8192) return {1, nch64, 4, 2};
        return {1, nch64, total_rows / 8 >= 1024 ? 8 : 4, 1};
    }
    B1XlShape sh{0, 0, 2, 2};
    switch (nch64) {
        case 6: sh.ks = 2; sh.ch = 3; break;
        case 8: sh.ks = 4; sh.ch = 2; break;
        case 12: sh.ks = 4; sh.ch = 3; break;
        default: return {0, 0, 0, 0};
    }
    if (total_rows / (sh.g * 2) < 512) sh.r = 1;
    return sh;
}

template <int MODE, int CH, int KS, int NW>
KernelFn pick_b1_xl_r(int r)
{
    return r == 2 ? q8_0_gemv_fast<MODE, 1, 2, CH, KS, true, NW> : q8_0_gemv_fast<MODE, 1, 1, CH, KS, true, NW>;
}

template <int MODE, int CH>
KernelFn pick_b1_xl_g(const B1XlShape& sh)
{
    if (sh.r == 2) return q8_0_gemv_fast<MODE, 1, 2, CH, 1, true, 4>;
    return sh.g == 8 ? q8_0_gemv_fast<MODE, 1, 1, CH, 1, true, 8> : q8_0_gemv_fast<MODE, 1, 1, CH, 1, true, 4>;
}

// SwiGLU (gate and up rows per output row): whole rows only, 4 row groups
// (2x8192x3072: 10.6-11.2 -> 10.1 us; 8 groups 10.2, 2 rows per wave 10.6).
KernelFn pick_b1_xl_swiglu(const B1XlShape& sh, int nch64)
{
    switch (nch64) {
        case 1: return pick_b1_xl_g<kSwiGLU, 1>(sh);
        case 2: return pick_b1_xl_g<kSwiGLU, 2>(sh);
        case 3: return pick_b1_xl_g<kSwiGLU, 3>(sh);
        case 4: return pick_b1_xl_g<kSwiGLU, 4>(sh);
        default: return nullptr;
    }
}

template <int MODE>
KernelFn pick_b1_xl(const B1XlShape& sh, int nch64)
{
    switch (nch64) {
        case 1: return pick_b1_xl_g<MODE, 1>(sh);
        case 2: return pick_b1_xl_g<MODE, 2>(sh);
        case 3: return pick_b1_xl_g<MODE, 3>(sh);
        case 4: return pick_b1_xl_g<MODE, 4>(sh);
        case 6: return pick_b1_xl_r<MODE, 3, 2, 4>(sh.r);
        case 8: return pick_b1_xl_r<MODE, 2, 4, 8>(sh.r);
        case 12: return pick_b1_xl_r<MODE, 3, 4, 8>(sh.r);
        default: return nullptr;
    }
}

// Largest x staged in LDS (bytes): up to 48 KB three workgroups still fit on a
// CU; beyond that the lost occupancy costs more than the L2 reads of x save
// (measured on the 8-row 3072-wide and 2-row 8192-wide cases).  Larger batch
// x width products read x from L2.
constexpr int64_t kXldsMax = 48 * 1024;

static_assert(kXldsMax <= 64 * 1024, "dynamic LDS above 64 KB would need a per-function opt-in");

template <int MODE>
KernelFn pick_general(int bt)
{
    switch (bt) {
        case 1: return q8_0_gemv_general<MODE, 1>;
        case 2: return q8_0_gemv_general<MODE, 2>;
        case 4: return q8_0_gemv_general<MODE, 4>;
        default: return q8_0_gemv_general<MODE, 8>;
    }
}

}  // namespace

bool q8_gemv_norm_fusable(const Q8GemvProblem& p)
{
    const int64_t nch = p.n_in / 16;
    return p.batch == 1 && nch % 64 == 0 && b1_shape((int)(nch / 64)).ks > 0;
}

hipError_t launch_q8_0_gemv(const Q8GemvProblem& p, hipStream_t s)
{
    if (p.norm_w && !q8_gemv_norm_fusable(p)) return hipErrorInvalidValue;   // only the one-row shape folds a norm
    Q8GemvArgs a = make_q8_gemv_args(p);

    // Batch rounds up to 1, 2, 4 or 8 (padding rows are never stored).
    const int bt = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
    const int nch64 = a.nch % 64 == 0 ? a.nch / 64 : 0;
    KernelFn fn = nullptr;
    int64_t blocks = 0;
    int threads = 256;
    bool xl = false;
    B1XlShape xsh = b1_xl_shape(nch64, a.total_rows);
    if (p.mode == kSwiGLU) xsh = xsh.ks == 1 ? B1XlShape{1, xsh.ch, 4, 1} : B1XlShape{0, 0, 0, 0};
    if (bt == 1 && xsh.ks > 0 && !p.norm_w && a.n_in * 4 <= kXldsMax) {
        switch (p.mode) {
            case kPlain: fn = pick_b1_xl<kPlain>(xsh, nch64); break;
            case kResidual: fn = pick_b1_xl<kResidual>(xsh, nch64); break;
            case kQKV: fn = pick_b1_xl<kQKV>(xsh, nch64); break;
            default: fn = pick_b1_xl_swiglu(xsh, nch64); break;
        }
        threads = 64 * xsh.ks * xsh.g;
        const int64_t rows_per_block = (int64_t)xsh.g * xsh.r;
        blocks = (a.total_rows + rows_per_block - 1) / rows_per_block;
        xl = true;
    } else if (bt == 2 && p.mode == kSwiGLU && nch64 >= 1 && nch64 <= 4 &&
               (int64_t)a.batch * a.n_in * 4 <= kXldsMax) {
        // two batch rows of SwiGLU: one gate/up row pair per wave, 8 row
        // groups sharing x in LDS (2x8192x3072: 11.4 -> 11.1 us against 2
        // row pairs per wave in 4 groups)
        switch (nch64) {
            case 1: fn = q8_0_gemv_fast<kSwiGLU, 2, 1, 1, 1, true, 8>; break;
            case 2: fn = q8_0_gemv_fast<kSwiGLU, 2, 1, 2, 1, true, 8>; break;
            case 3: fn = q8_0_gemv_fast<kSwiGLU, 2, 1, 3, 1, true, 8>; break;
            default: fn = q8_0_gemv_fast<kSwiGLU, 2, 1, 4, 1, true, 8>; break;
        }
        threads = 512;
        blocks = (a.total_rows + 7) / 8;
        xl = true;
    } else if (nch64 > 0 && bt == 1) {
        const B1Shape sh = b1_shape(nch64);
        const int r = b1_rows(p.mode, sh.ks, a.total_rows);
        switch (p.mode) {
            case kPlain: fn = pick_b1<kPlain>(r, nch64); break;
            case kResidual: fn = pick_b1<kResidual>(r, nch64); break;
            case kQKV: fn = pick_b1<kQKV>(r, nch64); break;
            default: fn = pick_b1<kSwiGLU>(r, nch64); break;
        }
        threads = 64 * sh.ks;
        blocks = (a.total_rows + r - 1) / r;
    } else if (nch64 > 0) {
        const int ks = split_ks(nch64);
        const int groups = 4 / ks;
        // largest R in {4, 2, 1} that still gives >= 512 workgroups
        int r = 4;
        while (r > 1 && a.total_rows / ((int64_t)groups * r) < 512) r >>= 1;
        xl = (int64_t)a.batch * a.n_in * 4 <= kXldsMax;
        switch (p.mode) {
            case kPlain: fn = pick_fast<kPlain>(bt, r, nch64, xl); break;
            case kResidual: fn = pick_fast<kResidual>(bt, r, nch64, xl); break;
            case kQKV: fn = pick_fast<kQKV>(bt, r, nch64, xl); break;
            default: fn = pick_fast<kSwiGLU>(bt, r, nch64, xl); break;
        }
        const int64_t rows_per_block = (int64_t)groups * fast_r(p.mode, bt, r);
        blocks = (a.total_rows + rows_per_block - 1) / rows_per_block;
    }
    if (!fn) {
        int lpr_log2 = 6;
        while (lpr_log2 > 1 && (1 << lpr_log2) > a.nch) --lpr_log2;
        a.lpr_log2 = lpr_log2;
        switch (p.mode) {
            case kPlain: fn = pick_general<kPlain>(bt); break;
            case kResidual: fn = pick_general<kResidual>(bt); break;
            case kQKV: fn = pick_general<kQKV>(bt); break;
            default: fn = pick_general<kSwiGLU>(bt); break;
        }
        const int64_t rows_per_wave = 64 >> lpr_log2;
        const int64_t waves = (a.total_rows + rows_per_wave - 1) / rows_per_wave;
        blocks = (waves + 3) / 4;
    }
    const size_t lds = xl ? (size_t)a.batch * (size_t)a.n_in * 4 : 0;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), lds, s, a);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
