// Q4_K dequant-GEMV for gfx950 (rustdoc "Module cuda_lane", Functions
// section: try_q4k_soa_gemv, on-device Q4_K dequant-GEMV over a repacked
// layout), batch 1..8.
//
// Super-block (256 weights, 144 bytes; the Q4_K workload definition that
// accompanies the pages): fp16 d, fp16 dmin, eight 6-bit scales and mins, 128
// nibble bytes.  In 64-element chunk p the low nibbles of qs[32p..32p+31] are
// sub-block 2p and the high nibbles sub-block 2p+1.  w = d*sc*q - dmin*m.  The
// repacked copy holds the nibbles, d|dmin, and the scales/mins unpacked to
// bytes (one word per sub-block pair), so no lane decodes the 6-bit packing.
//
// Work mapping: as the Q8_0 fast path, with an 8-byte chunk of nibbles per
// lane (16 weights: 8 of sub-block 2p, 8 of sub-block 2p+1), so a row of n_in
// weights is n_in/16 chunks and lane j of a wave takes chunks j, j+64, ...; K
// is split over KS waves of the workgroup and each wave computes R rows.  One
// batch row: x is copied once per workgroup into LDS (direct global->LDS
// loads before the weight loads, each chunk's 16 values gathered into one
// bank-swizzled 64-byte slot) and shared by several row groups; up to 4096
// columns a wave takes one whole row.  Measured against one chunk column per
// wave with x in registers (graph-replayed launches over rotated copies):
// 8192x3072 6.58 -> 6.06 us; more rows per wave were slower (the kernel is
// close to the VALU issue limit).  Wider rows keep x in registers: at
// 3072x8192 the LDS shapes measured 6.5-6.7 us against 6.53.  Per
// chunk the dot product is taken per sub-block in the factored form
//     sum_t w_t x_t = (d*sc) * sum_t q_t x_t - (dmin*m) * sum_t x_t,
// where d*sc and dmin*m are exact in f32.  sum_t x_t depends only on the lane's
// columns, so it is formed once per wave when x stays in registers.
#include "qdec_internal.h"

#include <algorithm>

namespace qdec {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

struct Q4KArgs {
    const uint8_t* qs;
    const uint32_t* dm;
    const uint32_t* sm;
    float* out;
    const float* x;
    int64_t n_in;
    int64_t n_out;
    int batch;
    int lpr_log2;  // general path: lanes per row group
    int nch;       // 8-byte nibble chunks per row = n_in / 16
};

__device__ inline u32x2 stream_load8(const uint8_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

__device__ inline uint32_t stream_load4(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// x values of chunk c: 8 for the low-nibble sub-block, 8 for the high one.
struct XChunk {
    float lo[8], hi[8];
    float slo, shi;  // their sums
};

__device__ inline int64_t chunk_x_offset(int c)
{
    const int sb = c >> 4, cc = c & 15;
    return (int64_t)sb * 256 + 64 * (cc >> 2) + 8 * (cc & 3);
}

__device__ inline void load_xchunk(const float* xrow, int c, XChunk& xc)
{
    const float4* pl = reinterpret_cast<const float4*>(xrow + chunk_x_offset(c));
    const float4* ph = reinterpret_cast<const float4*>(xrow + chunk_x_offset(c) + 32);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float4 v = pl[k], u = ph[k];
        xc.lo[4 * k] = v.x; xc.lo[4 * k + 1] = v.y; xc.lo[4 * k + 2] = v.z; xc.lo[4 * k + 3] = v.w;
        xc.hi[4 * k] = u.x; xc.hi[4 * k + 1] = u.y; xc.hi[4 * k + 2] = u.z; xc.hi[4 * k + 3] = u.w;
    }
}

__device__ inline void sum_xchunk(XChunk& xc)
{
    float a = xc.lo[0], b = xc.hi[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) {
        a += xc.lo[t];
        b += xc.hi[t];
    }
    xc.slo = a;
    xc.shi = b;
}

// Contribution of one 8-byte chunk (nibbles q, header words dm and sm) for x.
__device__ inline float chunk_dot(u32x2 q, uint32_t dm, uint32_t sm, const XChunk& xc, float acc)
{
    const float d = fp16_bits_to_f32((uint16_t)(dm & 0xffff));
    const float dmin = fp16_bits_to_f32((uint16_t)(dm >> 16));
    const float f_lo = d * (float)(sm & 0xff), f_hi = d * (float)((sm >> 8) & 0xff);
    const float g_lo = dmin * (float)((sm >> 16) & 0xff), g_hi = dmin * (float)(sm >> 24);
    const uint32_t w[2] = {q.x, q.y};
    float tl = 0.0f, th = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t lo = w[k] & 0x0f0f0f0fu;
        const uint32_t hi = (w[k] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            tl = __builtin_fmaf((float)((lo >> (8 * t)) & 0xffu), xc.lo[4 * k + t], tl);
            th = __builtin_fmaf((float)((hi >> (8 * t)) & 0xffu), xc.hi[4 * k + t], th);
        }
    }
    acc = __builtin_fmaf(f_lo, tl, acc);
    acc = __builtin_fmaf(-g_lo, xc.slo, acc);
    acc = __builtin_fmaf(f_hi, th, acc);
    acc = __builtin_fmaf(-g_hi, xc.shi, acc);
    return acc;
}

template <int CTRL>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wave (DPP within 16-lane rows, then the four row
// sums through scalar registers); the result is in every lane.
__device__ inline float wave_sum(float v)
{
    v += dpp<0x128>(v);
    v += dpp<0x124>(v);
    v += dpp<0x4E>(v);
    v += dpp<0xB1>(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// x staged in LDS (one batch row): chunk c's 16 values (8 of the low-nibble
// sub-block, 8 of the high one) as four float4, part q stored at float4 slot
// 4c + (q ^ ((c >> 1) & 3)) so that neighbouring lanes hit distinct banks.
__device__ inline const float* xchunk_src(const float* x, int c, int q)
{
    return x + chunk_x_offset(c) + (q < 2 ? 4 * q : 32 + 4 * (q - 2));
}

__device__ inline void lds_xchunk(const float* xs, int c, XChunk& xc)
{
    const float4* xp = reinterpret_cast<const float4*>(xs);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = xp[4 * c + (q ^ ((c >> 1) & 3))];
        float* d = q < 2 ? xc.lo + 4 * q : xc.hi + 4 * (q - 2);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
}

// Fast path: n_in a multiple of 1024; CH chunk columns per lane, KS waves per
// row group, R rows per wave, B batch rows; XL: x of one batch row staged in
// LDS (n_in floats of dynamic shared memory) and shared by the NW / KS row
// groups of the workgroup.
template <int B, int R, int CH, int KS, int NW, bool XL = false>
__global__ __launch_bounds__(64 * NW) void q4k_gemv_fast(Q4KArgs a)
{
    constexpr int GROUPS = NW / KS;
    static_assert(GROUPS * KS == NW, "whole row groups per workgroup");
    static_assert(!XL || B == 1, "LDS-staged x: one batch row");
    constexpr bool XREG = !XL && B * CH <= 4;
    __shared__ float part[KS > 1 ? NW : 1][R][B];
    extern __shared__ __attribute__((aligned(16))) float xs[];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = w / KS, ks = w % KS;
    const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + grp) * R;
    const int cbase = ks * CH;
    const int64_t nsb = a.n_in >> 8;

    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;

    if constexpr (XL) {
        const int nslot = (int)(a.n_in >> 2);
        for (int sb = w * 64; sb < nslot; sb += 64 * NW) {
            const int sl = sb + lane, c = sl >> 2, j = sl & 3;
            if (sl < nslot)
                __builtin_amdgcn_global_load_lds(xchunk_src(a.x, c, j ^ ((c >> 1) & 3)), (lds_void*)(xs + sb * 4), 16, 0, 0);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    XChunk xr[XREG ? CH : 1][XREG ? B : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
            for (int b = 0; b < B; ++b) load_xchunk(xrow[b], lane + 64 * (cbase + k), xr[k][b]);
    }

    // Row pointers: consecutive rows from the first when all R are in range
    // (short scalar set-up; the scalar unit is shared by the whole CU),
    // otherwise each row clamped alone.
    const uint8_t* qrow[R];
    const uint32_t* dmrow[R];
    const uint32_t* smrow[R];
    if (row0 + R <= a.n_out) {
        const uint8_t* q0 = a.qs + row0 * (a.n_in >> 1);
        const uint32_t* dm0 = a.dm + row0 * nsb;
        const uint32_t* sm0 = a.sm + row0 * nsb * 4;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qrow[r] = q0 + r * (a.n_in >> 1);
            dmrow[r] = dm0 + r * nsb;
            smrow[r] = sm0 + r * nsb * 4;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t rw = row0 + r;
            const int64_t rr = rw < a.n_out ? rw : a.n_out - 1;
            qrow[r] = a.qs + rr * (a.n_in >> 1);
            dmrow[r] = a.dm + rr * nsb;
            smrow[r] = a.sm + rr * nsb * 4;
        }
    }
    uint32_t dmv[CH][R], smv[CH][R];
    u32x2 qv[CH][R];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        const int c = lane + 64 * (cbase + k);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            dmv[k][r] = stream_load4(dmrow[r] + (c >> 4));
            smv[k][r] = stream_load4(smrow[r] + ((c >> 4) << 2) + ((c & 15) >> 2));
        }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r) qv[k][r] = stream_load8(qrow[r] + (int64_t)(lane + 64 * (cbase + k)) * 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XL) {
        // this wave's x slots have landed once at most the weight loads remain;
        // the barrier makes every wave's slots visible
        wait_vmcnt<3 * CH * R>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (XREG) {
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
            for (int b = 0; b < B; ++b) sum_xchunk(xr[k][b]);
    }

    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            XChunk xc;
            if constexpr (XREG) {
                xc = xr[XREG ? k : 0][XREG ? b : 0];
            } else if constexpr (XL) {
                lds_xchunk(xs, lane + 64 * (cbase + k), xc);
                sum_xchunk(xc);
            } else {
                load_xchunk(xrow[b], lane + 64 * (cbase + k), xc);
                sum_xchunk(xc);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][b] = chunk_dot(qv[k][r], dmv[k][r], smv[k][r], xc, acc[r][b]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = wave_sum(acc[r][b]);

    // lane l < R*B ends up with the (row l / B, batch row l % B) value
    float v = 0.0f;
    if constexpr (KS > 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) part[w][r][b] = acc[r][b];
        }
        __syncthreads();
        if (ks != 0) return;
        if (lane < R * B) {
#pragma unroll
            for (int k = 0; k < KS; ++k) v += part[w + k][lane / B][lane % B];
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
                if (lane == r * B + b) v = acc[r][b];
    }
    const int rl = lane / B, bl = lane % B;
    if (lane < R * B && bl < a.batch && row0 + rl < a.n_out) a.out[(int64_t)bl * a.n_out + row0 + rl] = v;
}

// General path: row groups of LPR lanes, bounds-checked chunk loop.
template <int B>
__global__ __launch_bounds__(256) void q4k_gemv_general(Q4KArgs a)
{
    const int lpr = 1 << a.lpr_log2;
    const int lane = threadIdx.x & 63;
    const int g = lane >> a.lpr_log2;
    const int j = lane & (lpr - 1);
    const int groups = 64 >> a.lpr_log2;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nsb = a.n_in >> 8;
    const int64_t row = wave * groups + g;
    const int64_t rr = row < a.n_out ? row : a.n_out - 1;
    const uint8_t* qrow = a.qs + rr * (a.n_in >> 1);
    const uint32_t* dmrow = a.dm + rr * nsb;
    const uint32_t* smrow = a.sm + rr * nsb * 4;
    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    for (int c = j; c < a.nch; c += lpr) {
        const uint32_t dm = stream_load4(dmrow + (c >> 4));
        const uint32_t sm = stream_load4(smrow + ((c >> 4) << 2) + ((c & 15) >> 2));
        const u32x2 q = stream_load8(qrow + (int64_t)c * 8);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            XChunk xc;
            load_xchunk(xrow[b], c, xc);
            sum_xchunk(xc);
            acc[b] = chunk_dot(q, dm, sm, xc, acc[b]);
        }
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) {
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] += __shfl_xor(acc[b], off);
    }
    if (j != 0 || row >= a.n_out) return;
#pragma unroll
    for (int b = 0; b < B; ++b)
        if (b < a.batch) a.out[(int64_t)b * a.n_out + row] = acc[b];
}

using KernelFn = void (*)(Q4KArgs);
using KernelFnT = void (*)(Q4KTView, const float*, int64_t, int64_t, float*);

template <int B, int R>
KernelFn pick_split(int nch64)
{
    switch (nch64) {
        case 1: return q4k_gemv_fast<B, R, 1, 1, 4>;
        case 2: return q4k_gemv_fast<B, R, 2, 1, 4>;
        case 3: return q4k_gemv_fast<B, R, 3, 1, 4>;
        case 4: return q4k_gemv_fast<B, R, 2, 2, 4>;
        case 6: return q4k_gemv_fast<B, R, 3, 2, 4>;
        case 8: return q4k_gemv_fast<B, R, 2, 4, 4>;
        case 12: return q4k_gemv_fast<B, R, 3, 4, 4>;
        case 16: return q4k_gemv_fast<B, R, 4, 4, 4>;
        default: return nullptr;
    }
}

int split_ks(int nch64) { return nch64 <= 3 ? 1 : (nch64 <= 6 ? 2 : 4); }

// One batch row: one chunk column per wave (two above 8192 columns) and one
// row group per workgroup, as the Q8_0 path, so the arithmetic left after a
// wave's last load stays short.
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

// One batch row with x in LDS (up to 4096 columns): one whole row per wave,
// G = 8 row groups per workgroup, 4 while that leaves fewer than 1024
// workgroups.
struct B1XlShape { int ks, ch, g, r; };

B1XlShape b1_xl_shape(int nch64, int64_t n_out)
{
    if (nch64 >= 1 && nch64 <= 4) return {1, nch64, n_out / 8 >= 1024 ? 8 : 4, 1};
    return {0, 0, 0, 0};
}

template <int CH>
KernelFn pick_b1_xl_g(int g)
{
    return g == 8 ? q4k_gemv_fast<1, 1, CH, 1, 8, true> : q4k_gemv_fast<1, 1, CH, 1, 4, true>;
}

KernelFn pick_b1_xl(const B1XlShape& sh, int nch64)
{
    switch (nch64) {
        case 1: return pick_b1_xl_g<1>(sh.g);
        case 2: return pick_b1_xl_g<2>(sh.g);
        case 3: return pick_b1_xl_g<3>(sh.g);
        case 4: return pick_b1_xl_g<4>(sh.g);
        default: return nullptr;
    }
}

template <int R>
KernelFn pick_b1_split(int nch64)
{
    switch (nch64) {
        case 1: return q4k_gemv_fast<1, R, 1, 1, 1>;
        case 2: return q4k_gemv_fast<1, R, 1, 2, 2>;
        case 3: return q4k_gemv_fast<1, R, 1, 3, 3>;
        case 4: return q4k_gemv_fast<1, R, 1, 4, 4>;
        case 6: return q4k_gemv_fast<1, R, 1, 6, 6>;
        case 8: return q4k_gemv_fast<1, R, 1, 8, 8>;
        case 12: return q4k_gemv_fast<1, R, 2, 6, 6>;
        case 16: return q4k_gemv_fast<1, R, 2, 8, 8>;
        default: return nullptr;
    }
}

// ------------------------------------------------------ matrix cores --
// One batch row on the integer matrix cores.  A 512-byte tile of the tiled
// copy is 16 rows x one 64-weight chunk c of the row (low nibbles: sub-block
// 2c, high nibbles: 2c+1), one K = 64 step of v_mfma_i32_16x16x64_i8: a lane's
// 8 bytes, masked to their low and high nibbles, are its 16 B operand bytes
// as they stand (the nibbles 0..15 are int8 values).
// x is written as a fixed-point number per sub-block b of 32 values:
// X_k = trunc(x_k * 2^(30 - e_b)), |x_k| < 2^e_b for every k of the block, so
// |X_k| < 2^30 and x_k = X_k 2^(e_b - 30) + eps_k, |eps_k| < 2^(e_b - 30) (zero
// whenever |x_k| >= 2^(e_b - 6): the 24-bit significand then fits).  X_k has
// the signed base-256 digits X = a3 2^24 + a2 2^16 + a1 2^8 + a0, a_j in
// -128..127 (the bytes of X + 0x80808080, each less 0x80), each an int8.  The
// A operand's rows are (half h, digit j) = 4h + j: digit j of the sub-block
// 2c + h values, zero on the other half's k-slots, so the MFMA returns in
// exact int32, per weight row r and sub-block 2c + h, D_j = sum_k q_k a_j,k
// (|D_j| <= 32*15*128); rows 8..15 repeat rows 0..7.  Lane r + 16h then forms
// sum_k q_k X_k = (256 D3 + D2) 2^16 + (256 D1 + D0) (both brackets exact
// integers below 2^24, one rounding in the fma) and accumulates, as in the
// factored Q4_K form,
//     (d sc) * (2^(e_b - 30) sum_k q_k X_k) - (dmin m) * sum_k x_k,
// d sc exact (11 x 6 significant bits), the power-of-two scaling exact, sum_k
// x_k the f32 sum of the sub-block's 32 values in a fixed order.
// A workgroup is RG 16-row groups, each with K split over KS waves of T
// chunks (T % 4 == 0, so a wave starts on a super-block; T even, for the
// tile pairs below).  Each thread loads 4 values of x (a quad; two when
// n_in/4 > threads) and waits for them, then issues every weight load of its
// wave (T tiles, per tile pair the scale words, per super-block d|dmin);
// while those are in flight the workgroup writes to LDS the A operands of
// every chunk (512 bytes: rows 0..7 x 4 k-groups x 16 bytes) and, per
// sub-block, the sum of x and e_b - 30, found with DPP over the sub-block's 8
// consecutive quads.
// Error per output, beyond the f32 rounding of the VALU kernel: at most
// 2^(e_b - 30) <= 2^-29 max_b |x| per x value, times sum_k d sc q_k.
template <int KS, int T, int RG>
__global__ __launch_bounds__(64 * KS * RG) void q4k_gemv_mfma(Q4KTView w, const float* __restrict__ x,
                                                              int64_t n_in, int64_t n_out, float* __restrict__ out)
{
    static_assert(T % 4 == 0 && T >= 4 && T <= 16 && KS * RG <= 16, "T chunks per wave, KS * RG waves");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int n = 64 * T * KS;     // n_in
    constexpr int NT = 64 * KS * RG;   // threads
    constexpr int NQ = n / 4;          // quads of x
    constexpr int QK = (NQ + NT - 1) / NT;
    static_assert(QK <= 4, "quads per thread");
    // A operands (512 bytes a chunk); per sub-block the sum of x and e_b - 30
    __shared__ __attribute__((aligned(16))) uint8_t lds[8 * n];
    __shared__ float2 xsc[n / 32];
    __shared__ float red[RG][KS][16];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wv / KS, kw = wv % KS;
    const int64_t groups = q4kt_groups(n_out);
    const int64_t Gw = (int64_t)blockIdx.x * RG + rg;          // this wave's row group
    const int64_t G = Gw < groups ? Gw : groups - 1;           // a spare wave reads the last one
    const int64_t nch = n_in >> 6, nsb = n_in >> 8;
    const int c0 = kw * T;   // first chunk of this wave, a multiple of 4

    // quads i = tid + k NT of x, live for whole waves (NQ % 64 == 0)
    float4 xv[QK];
#pragma unroll
    for (int k = 0; k < QK; ++k)
        xv[k] = 64 * wv + k * NT < NQ ? reinterpret_cast<const float4*>(x)[tid + k * NT]
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    // x first: every workgroup reads it, and behind the weight requests of
    // the whole grid it would land late
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
    // every weight load of this wave: the tiles, per tile pair the scale
    // words of row lane % 16 for tile 2p + lane / 32, per super-block d|dmin
    u32x2 qv[T];
    uint32_t smv[T / 2], dmv[T / 4];
    {
        const u32x2* qt = reinterpret_cast<const u32x2*>(w.q) + (G * nch + c0) * 64 + lane;
        const uint32_t* st = w.sm + (G * nch + c0 + (lane >> 5)) * 16 + (lane & 15);
        const uint32_t* dt = w.dm + (G * nsb + c0 / 4) * 16 + (lane & 15);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            qv[t] = __builtin_nontemporal_load(qt + t * 64);
            if (t % 2 == 0) smv[t / 2] = __builtin_nontemporal_load(st + t * 16);
            if (t % 4 == 0) dmv[t / 4] = __builtin_nontemporal_load(dt + (t / 4) * 16);
        }
    }
    asm volatile("" ::: "memory");
    // A operands, sums and scales of x: quad i holds values 4i .. 4i + 3, of
    // sub-block i / 8, chunk c = i / 16, half h, k-group g, half-run hr
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        if (64 * wv + k * NT >= NQ) break;
        const int i = tid + k * NT;
        const float v[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
        uint32_t amax = max(max(__builtin_bit_cast(uint32_t, v[0]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[1]) & 0x7fffffffu),
                            max(__builtin_bit_cast(uint32_t, v[2]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[3]) & 0x7fffffffu));
        float sum = ((v[0] + v[1]) + v[2]) + v[3];
        // over the sub-block's 8 quads (8 consecutive lanes): lane ^ 1, lane ^ 2
        // (quad permutes), then lane i <-> 7 - i (half-row mirror)
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x141, 0xF, 0xF, false));
        sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));
        sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
        sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x141, 0xF, 0xF, false));
        // amax = m 2^e with 0.5 <= m < 1, so every |x| < 2^e (e = 0 for zeros)
        const int e_b = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, amax));
        // X = trunc(x 2^(30 - e)), |X| < 2^30; its signed base-256 digits are
        // the bytes of X + 0x80808080, each less 0x80 (a non-finite sub-block
        // converts zeros: its sum below makes every output NaN, and an
        // infinity or NaN has no defined int conversion; a select per value
        // measured cheaper here than a wave-uniform branch per quad)
        const bool fin = amax < 0x7f800000u;
        uint32_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = (uint32_t)(int)(fin ? __builtin_amdgcn_ldexpf(v[e], 30 - e_b) : 0.0f) + 0x80808080u;
        // transpose: word j = digit j of the 4 values
        uint32_t wd[4];
        {
            const uint32_t t01l = __builtin_amdgcn_perm(y[1], y[0], 0x05010400u);
            const uint32_t t01h = __builtin_amdgcn_perm(y[1], y[0], 0x07030602u);
            const uint32_t t23l = __builtin_amdgcn_perm(y[3], y[2], 0x05010400u);
            const uint32_t t23h = __builtin_amdgcn_perm(y[3], y[2], 0x07030602u);
            wd[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u) ^ 0x80808080u;
            wd[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u) ^ 0x80808080u;
            wd[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u) ^ 0x80808080u;
            wd[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u) ^ 0x80808080u;
        }
        // A row 4h + j, k-group g of chunk c: bytes 8h + 4hr take digit j of
        // the quad, bytes 8(1 - h) + 4hr zeros
        const int c = i >> 4, h = (i >> 3) & 1, g = (i >> 1) & 3, hr = i & 1;
        uint8_t* cell = lds + 512 * c + 16 * (4 * (4 * h) + g) + 4 * hr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint32_t*>(cell + 64 * j + 8 * h) = wd[j];
            *reinterpret_cast<uint32_t*>(cell + 64 * j + 8 - 8 * h) = 0u;
        }
        // a non-finite x makes its sub-block's sum, and so the output, NaN
        if ((i & 7) == 0)
            xsc[i >> 3] = make_float2(amax < 0x7f800000u ? sum : __builtin_nanf(""),
                                      __builtin_bit_cast(float, e_b - 30));
    }
    __syncthreads();

    // A operand of lane (row m = lane % 16, k-group g = lane / 16): 16 bytes
    // of row m % 8
    const int aoff = 512 * c0 + 16 * (4 * (lane & 7) + (lane >> 4));
    // D side, per tile pair (2p, 2p + 1): the results of both MFMAs have
    // rows 8..15 (lanes 32..63) equal to rows 0..7 (lanes 0..31); a lane swap
    // puts tile 2p in lanes 0..31 and tile 2p + 1 in lanes 32..63, so lane
    // r + 16 hd + 32 tp holds sub-block 2c + hd of row r, c = c0 + 2p + tp
    const int hd = (lane >> 4) & 1, tp = lane >> 5, sh = 8 * hd;
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < T / 2; ++p) {
        i32x4 D[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int t = 2 * p + k;
            const i32x4 A = *reinterpret_cast<const i32x4*>(lds + aoff + 512 * t);
            const i32x4 B = {(int)(qv[t][0] & 0x0f0f0f0fu), (int)(qv[t][1] & 0x0f0f0f0fu),
                             (int)((qv[t][0] >> 4) & 0x0f0f0f0fu), (int)((qv[t][1] >> 4) & 0x0f0f0f0fu)};
            D[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
        }
        int Dp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // lanes 32..63 of D[0] (equal to its lanes 0..31) trade places with
            // lanes 0..31 of D[1]
            const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)D[0][e], (unsigned)D[1][e], false, false);
            Dp[e] = (int)sw[0];
        }
        const int c = c0 + 2 * p + tp;
        const float u = __builtin_fmaf((float)(Dp[3] * 256 + Dp[2]), 65536.0f, (float)(Dp[1] * 256 + Dp[0]));
        const uint32_t dm = dmv[p / 2];
        const float d = fp16_bits_to_f32((uint16_t)(dm & 0xffff));
        const float dmin = fp16_bits_to_f32((uint16_t)(dm >> 16));
        const uint32_t smh = smv[p] >> sh;
        const float sc = (float)(smh & 0xffu), mn = (float)((smh >> 16) & 0xffu);
        const float2 xb = xsc[2 * c + hd];
        // u 2^(e_b - 30) is exact (in range for any normal x); d sc is exact
        acc = __builtin_fmaf(d * sc, __builtin_amdgcn_ldexpf(u, __builtin_bit_cast(int, xb.y)), acc);
        acc = __builtin_fmaf(-(dmin * mn), xb.x, acc);
    }
    // row r: its sub-block halves and tiles in lanes r + 16 hd + 32 tp, then
    // the KS waves of its group in order
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    if constexpr (KS > 1) {
        if (lane < 16) red[rg][kw][lane] = acc;
        __syncthreads();
        if (kw != 0) return;
        if (lane < 16) {
            float s2 = red[rg][0][lane];
#pragma unroll
            for (int k = 1; k < KS; ++k) s2 += red[rg][k][lane];
            acc = s2;
        }
    }
    const int64_t row = Gw * 16 + lane;
    if (lane < 16 && Gw < groups && row < n_out) out[row] = acc;
}

// K split: n_in = 64 KS T, T = 8, 12 or 16 chunks a wave: 1024 on 2 waves,
// 2048 .. 4096 on 4, 6144 and 8192 on 8.  Two row groups share a workgroup
// (and its x operands) when that still leaves 256 workgroups.
bool q4k_mfma_shape(int64_t n_in, int* ks, int* t)
{
    switch (n_in) {
        case 1024: *ks = 2; *t = 8; return true;
        case 2048: *ks = 4; *t = 8; return true;
        case 3072: *ks = 4; *t = 12; return true;
        case 4096: *ks = 4; *t = 16; return true;
        case 6144: *ks = 8; *t = 12; return true;
        case 8192: *ks = 8; *t = 16; return true;
        default: return false;
    }
}

template <int KS, int T>
KernelFnT q4k_mfma_pick(int rg)
{
    return rg == 2 ? q4k_gemv_mfma<KS, T, 2> : q4k_gemv_mfma<KS, T, 1>;
}

// 2..8 batch rows on the integer matrix cores from the same tiled copy, one
// v_mfma_i32_16x16x32_i8 per 32-value sub-block and fragment of 4 batch rows:
// the B operand is the lane's 8 nibble bytes masked to their low (sub-block
// 2c) or high (2c + 1) nibbles, which are its 8 k-values of that sub-block as
// they stand; the A operand stacks 4 batch rows x 4 digits of x as a 30-bit
// fixed-point number per (batch row, sub-block), as the one-row kernel does
// per sub-block.  Lane n + 16 b' of fragment f receives the four digit sums of
// batch row 4 f + b' and weight row n, forms u = (256 D3 + D2) 2^16 + (256 D1
// + D0) and accumulates (d sc) u 2^(e - 30) - (dmin m) sum_k x_k, the sum of
// the sub-block's 32 values taken once per workgroup in a fixed order.  A
// workgroup holds the A operands of whole rows (batch x n_in x 4 bytes of
// LDS, at most 96 KB), RG row groups x KS waves of T chunks of 64 values.
// The A cells are XOR-swizzled by sub-block inside each 16-lane group (as in
// the Q8_0 kernel: conflict-free reads, spread writes).  A non-finite x makes
// every output of its batch row NaN (through its sub-block sum).
template <int KS, int T, int NV, int RG>
__global__ __launch_bounds__(64 * KS * RG) void q4k_gemv_rows(Q4KTView w, const float* __restrict__ x, int64_t n_in,
                                                             int64_t n_out, int batch, float* __restrict__ out)
{
    static_assert(KS * RG <= 16 && T % 4 == 0 && NV >= 1 && NV <= 2, "KS * RG waves, T chunks a wave");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int NCH = KS * T;                 // 64-value chunks of a row
    constexpr int NB = 2 * NCH;                 // 32-value sub-blocks of a row
    constexpr int NW = KS * RG;
    constexpr int NT = 64 * NW;
    constexpr int XB = NB * NV * 512;           // A fragments
    constexpr int RB = NW * NV * 64 * 4;        // wave sums, after the products
    constexpr int LB = XB > RB ? XB : RB;
    constexpr int IPT = (4 * NV * NB * 4 + NT - 1) / NT;   // x items (8 values) a thread
    static_assert(IPT <= 8, "x items per thread");
    __shared__ __attribute__((aligned(16))) char lds[LB];
    __shared__ __attribute__((aligned(16))) int xe[4 * NV][NB];     // e - 30 per (batch row, sub-block)
    __shared__ __attribute__((aligned(16))) float xsum[4 * NV][NB]; // sum of the sub-block's x

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wv / KS, kw = wv % KS;
    const int64_t groups = q4kt_groups(n_out);
    const int64_t Gw = (int64_t)blockIdx.x * RG + rg;
    const int64_t G = Gw < groups ? Gw : groups - 1;     // a spare wave reads the last group
    const int64_t nsb = n_in >> 8;
    const int c0 = kw * T;                               // first chunk of this wave

    // x item it = (b, blk, g), g fastest: values 32 blk + 8 g .. +7 of batch row b
    const int items = batch * NB * 4;
    float4 xv[IPT][2];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {
            const float4* src = reinterpret_cast<const float4*>(x + (int64_t)(it / (NB * 4)) * n_in) + 2 * (it % (NB * 4));
            xv[j][0] = src[0];
            xv[j][1] = src[1];
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): x before the weight requests queue up
    asm volatile("" ::: "memory");
    // every weight load of this wave: the chunk tiles, their scale words
    // (row lane % 16) and per super-block d|dmin
    u32x2 qv[T];
    uint32_t smv[T], dmv[T / 4];
    {
        const u32x2* qt = reinterpret_cast<const u32x2*>(w.q) + (G * NCH + c0) * 64 + lane;
        const uint32_t* st = w.sm + (G * NCH + c0) * 16 + (lane & 15);
        const uint32_t* dt = w.dm + (G * nsb + c0 / 4) * 16 + (lane & 15);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            qv[t] = __builtin_nontemporal_load(qt + t * 64);
            smv[t] = __builtin_nontemporal_load(st + t * 16);
            if (t % 4 == 0) dmv[t / 4] = __builtin_nontemporal_load(dt + (t / 4) * 16);
        }
    }
    asm volatile("" ::: "memory");

    // A fragments: lane (m, g) of fragment (blk, f) reads the 8 bytes at
    // ((blk NV + f) 64 + 16 g + (m ^ (blk % 16))) * 8 -- digit m % 4 of batch
    // row 4 f + m / 4 at k = 8 g .. 8 g + 7 of sub-block blk
    u32x2* xf = reinterpret_cast<u32x2*>(lds);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int it = (int)threadIdx.x + j * NT;
        if (it < items) {   // the 4 lanes of a sub-block agree
            const int b = it / (NB * 4), blk = (it >> 2) % NB, g = it & 3;
            float v[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                          xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
            uint32_t amax = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = max(amax, __builtin_bit_cast(uint32_t, v[e]) & 0x7fffffffu);
            float sum = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
            // over the sub-block's 4 items (4 consecutive lanes): lane ^ 1, lane ^ 2
            amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
            amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
            const bool fin = amax < 0x7f800000u;
            if (__builtin_amdgcn_ballot_w64(!fin) != 0) {
                // rare: a non-finite sub-block converts zeros; its sum (made
                // NaN below) carries the NaN to every output of the row
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fin ? v[e] : 0.0f;
            }
            // amax = m 2^e with 0.5 <= m < 1, so every |x| < 2^e (e = 0 for zeros)
            const int ex = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, amax));
            uint32_t y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (uint32_t)(int)__builtin_amdgcn_ldexpf(v[e], 30 - ex) + 0x80808080u;
            uint32_t dg[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t t01l = __builtin_amdgcn_perm(y[4 * h + 1], y[4 * h], 0x05010400u);
                const uint32_t t01h = __builtin_amdgcn_perm(y[4 * h + 1], y[4 * h], 0x07030602u);
                const uint32_t t23l = __builtin_amdgcn_perm(y[4 * h + 3], y[4 * h + 2], 0x05010400u);
                const uint32_t t23h = __builtin_amdgcn_perm(y[4 * h + 3], y[4 * h + 2], 0x07030602u);
                dg[h][0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u) ^ 0x80808080u;
                dg[h][1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u) ^ 0x80808080u;
                dg[h][2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u) ^ 0x80808080u;
                dg[h][3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u) ^ 0x80808080u;
            }
            u32x2* frag = xf + (blk * NV + (b >> 2)) * 64 + 16 * g;
#pragma unroll
            for (int dj = 0; dj < 4; ++dj) frag[(4 * (b & 3) + dj) ^ (blk & 15)] = u32x2{dg[0][dj], dg[1][dj]};
            if (g == 0) {
                xe[b][blk] = ex - 30;
                xsum[b][blk] = fin ? sum : __builtin_nanf("");
            }
        }
    }
    __syncthreads();   // LDS only: the weight loads stay in flight

    // lane (n = lane % 16, b' = lane / 16) of fragment f: batch row 4 f + b';
    // sub-block blk = 2 (c0 + t) + h
    const int b4 = lane >> 4;
    float acc[NV];
#pragma unroll
    for (int f = 0; f < NV; ++f) acc[f] = 0.0f;
    const u32x2* xw = xf + 2 * c0 * NV * 64;
    int4 e4[NV];
    float4 s4[NV];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t % 2 == 0) {
            // exponents and sums of sub-blocks 2 (c0 + t) .. +3 (t even)
#pragma unroll
            for (int f = 0; f < NV; ++f) {
                e4[f] = *reinterpret_cast<const int4*>(&xe[4 * f + b4][2 * (c0 + t)]);
                s4[f] = *reinterpret_cast<const float4*>(&xsum[4 * f + b4][2 * (c0 + t)]);
            }
        }
        const uint32_t dm = dmv[t / 4];
        const float d = fp16_bits_to_f32((uint16_t)(dm & 0xffff));
        const float dmin = fp16_bits_to_f32((uint16_t)(dm >> 16));
        const uint32_t smw = smv[t];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int lb = 2 * t + h;   // sub-block within the wave's range
            const float dsc = d * (float)((smw >> (8 * h)) & 0xffu);
            const float dmm = dmin * (float)((smw >> (16 + 8 * h)) & 0xffu);
            const u32x2 Bq = {(h ? (qv[t][0] >> 4) : qv[t][0]) & 0x0f0f0f0fu, (h ? (qv[t][1] >> 4) : qv[t][1]) & 0x0f0f0f0fu};
            const int sl = lane ^ ((2 * (c0 + t) + h) & 15);
#pragma unroll
            for (int f = 0; f < NV; ++f) {
                const u32x2 A = xw[(lb * NV + f) * 64 + sl];
                const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, A),
                                                                      __builtin_bit_cast(long, Bq),
                                                                      i32x4{0, 0, 0, 0}, 0, 0, 0);
                const float u = __builtin_fmaf((float)(D[3] * 256 + D[2]), 65536.0f, (float)(D[1] * 256 + D[0]));
                const int q2 = (t % 2) * 2 + h;   // position of sub-block lb in the 4 read above
                const int eb = q2 == 0 ? e4[f].x : q2 == 1 ? e4[f].y : q2 == 2 ? e4[f].z : e4[f].w;
                const float sx = q2 == 0 ? s4[f].x : q2 == 1 ? s4[f].y : q2 == 2 ? s4[f].z : s4[f].w;
                acc[f] = __builtin_fmaf(dsc, __builtin_amdgcn_ldexpf(u, eb), acc[f]);
                acc[f] = __builtin_fmaf(-dmm, sx, acc[f]);
            }
        }
    }

    // the KS wave sums of each output in wave order, then the store
    __syncthreads();   // every wave is done with the A fragments
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int f = 0; f < NV; ++f) red[(wv * NV + f) * 64 + lane] = acc[f];
    __syncthreads();
    if (kw != 0) return;
    const int64_t row = Gw * 16 + (lane & 15);
#pragma unroll
    for (int f = 0; f < NV; ++f) {
        float sm = red[((rg * KS) * NV + f) * 64 + lane];
#pragma unroll
        for (int k = 1; k < KS; ++k) sm += red[((rg * KS + k) * NV + f) * 64 + lane];
        const int b = 4 * f + b4;
        if (b < batch && Gw < groups && row < n_out) out[(int64_t)b * n_out + row] = sm;
    }
}

// Shapes of the rows kernel: n_in = 64 KS T with T = 8 chunks a wave; whole
// rows of up to 8 batch rows to 4096 columns (6144 and 8192 up to 4 rows).
bool q4k_rows_shape(int64_t n_in, int64_t batch, int* ks)
{
    switch (n_in) {
        case 1024: *ks = 2; return true;
        case 2048: *ks = 4; return true;
        case 3072: *ks = 6; return true;
        case 4096: *ks = 8; return true;
        case 6144: *ks = 12; return batch <= 4;
        case 8192: *ks = 16; return batch <= 4;
        default: return false;
    }
}

int q4k_rows_rg(int64_t groups, int ks) { return groups >= 512 && ks <= 6 ? 2 : 1; }

using KernelFnR4 = void (*)(Q4KTView, const float*, int64_t, int64_t, int, float*);

template <int KS>
KernelFnR4 q4k_rows_pick_nv(int nv, int rg)
{
    if constexpr (KS <= 6) {
        if (rg == 2) return nv == 1 ? q4k_gemv_rows<KS, 8, 1, 2> : q4k_gemv_rows<KS, 8, 2, 2>;
    }
    if constexpr (KS <= 8) return nv == 1 ? q4k_gemv_rows<KS, 8, 1, 1> : q4k_gemv_rows<KS, 8, 2, 1>;
    return nv == 1 ? q4k_gemv_rows<KS, 8, 1, 1> : nullptr;
}

KernelFnR4 q4k_rows_pick(int ks, int nv, int rg)
{
    switch (ks) {
        case 2: return q4k_rows_pick_nv<2>(nv, rg);
        case 4: return q4k_rows_pick_nv<4>(nv, rg);
        case 6: return q4k_rows_pick_nv<6>(nv, rg);
        case 8: return q4k_rows_pick_nv<8>(nv, rg);
        case 12: return q4k_rows_pick_nv<12>(nv, rg);
        case 16: return q4k_rows_pick_nv<16>(nv, rg);
        default: return nullptr;
    }
}

}  // namespace

// 5..8 rows at 6144 and 8192 columns (whose A cells would not fit one
// workgroup's LDS) run as two launches of (batch + 1) / 2 and the remaining
// rows, each 2..4 rows, on x and out offset by the first part's rows.
bool q4k_rows_split(int64_t n_in, int64_t batch)
{
    return batch > 4 && batch <= 8 && (n_in == 6144 || n_in == 8192);
}

bool q4k_mfma_supported(int64_t n_in, int64_t batch)
{
    int ks = 0, t = 0;
    if (batch == 1) return q4k_mfma_shape(n_in, &ks, &t);
    if (q4k_rows_split(n_in, batch)) return true;
    return batch >= 2 && batch <= 8 && q4k_rows_shape(n_in, batch, &ks);
}

std::string q4k_mfma_plan_check(int64_t n_in, int64_t n_out, int64_t batch)
{
    if (q4k_rows_split(n_in, batch)) {
        const int64_t b0 = (batch + 1) / 2;
        const std::string e = q4k_mfma_plan_check(n_in, n_out, b0);
        return e.empty() ? q4k_mfma_plan_check(n_in, n_out, batch - b0) : e;
    }
    int ks = 0, t = 0;
    const int64_t groups = q4kt_groups(n_out), nch = n_in / 64, nsb = n_in / 256;
    int64_t grid = 0, rg = 1, tt = 0;
    if (batch == 1) {
        if (!q4k_mfma_shape(n_in, &ks, &t) || 64LL * ks * t != n_in) return "q4k matrix-core GEMV: unsupported width";
        rg = groups >= 512 ? 2 : 1;
        tt = t;
    } else {
        if (!q4k_rows_shape(n_in, batch, &ks) || 64LL * ks * 8 != n_in) return "q4k rows GEMV: unsupported shape";
        rg = q4k_rows_rg(groups, ks);
        tt = 8;
        const int64_t nv = (batch + 3) / 4, nb = 2 * nch;
        if (nb * nv * 512 + 2 * 4 * nv * nb * 4 > 160 * 1024) return "q4k rows GEMV: LDS";
        // x: items (b, blk, g) below batch nb 4 read floats b n_in + 32 blk + 8 g .. +7
        if ((int64_t)(4 * nv * nb * 4 + 64 * ks * rg - 1) / (64 * ks * rg) > 8) return "q4k rows GEMV: x items per thread";
    }
    grid = (groups + rg - 1) / rg;
    if (grid <= 0 || grid > 0x7fffffffLL) return "q4k matrix-core GEMV: grid out of range";
    const int64_t g_last = std::min<int64_t>(grid * rg - 1, groups - 1);
    const int64_t q_end = ((g_last * nch + (int64_t)(ks - 1) * tt + tt - 1) * 64 + 63) * 8 + 8;
    const int64_t sm_end = ((g_last * nch + (int64_t)(ks - 1) * tt + tt - 1) * 16 + 15) * 4 + 4;
    const int64_t dm_end = ((g_last * nsb + nsb - 1) * 16 + 15) * 4 + 4;
    if (q_end > groups * nch * 512 || sm_end > groups * nch * 64 || dm_end > groups * nsb * 64)
        return "q4k matrix-core GEMV: a weight read runs past the tiled copy";
    return "";
}

hipError_t launch_q4k_gemv_mfma(Q4KTView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                                hipStream_t s)
{
    int ks = 0, t = 0;
    if (!q4k_mfma_plan_check(n_in, n_out, batch).empty()) return hipErrorInvalidConfiguration;
    if (q4k_rows_split(n_in, batch)) {
        const int64_t b0 = (batch + 1) / 2;
        const hipError_t e = launch_q4k_gemv_mfma(w, n_in, n_out, b0, x, out, s);
        if (e != hipSuccess) return e;
        return launch_q4k_gemv_mfma(w, n_in, n_out, batch - b0, x + b0 * n_in, out + b0 * n_out, s);
    }
    if (batch > 1) {
        if (!q4k_rows_shape(n_in, batch, &ks)) return hipErrorNotSupported;
        const int64_t groups = q4kt_groups(n_out);
        const int rg = q4k_rows_rg(groups, ks), nv = (int)((batch + 3) / 4);
        const KernelFnR4 fr = q4k_rows_pick(ks, nv, rg);
        if (!fr) return hipErrorNotSupported;
        hipLaunchKernelGGL(fr, dim3((unsigned)((groups + rg - 1) / rg)), dim3(64 * ks * rg), 0, s, w, x, n_in, n_out,
                           (int)batch, out);
        count_launch();
        return hipGetLastError();
    }
    if (!q4k_mfma_shape(n_in, &ks, &t)) return hipErrorNotSupported;
    const int64_t groups = q4kt_groups(n_out);
    const int rg = groups >= 512 ? 2 : 1;
    KernelFnT fn = ks == 2 ? q4k_mfma_pick<2, 8>(rg)
                 : ks == 4 ? (t == 8 ? q4k_mfma_pick<4, 8>(rg) : t == 12 ? q4k_mfma_pick<4, 12>(rg)
                                                                         : q4k_mfma_pick<4, 16>(rg))
                           : (t == 12 ? q4k_mfma_pick<8, 12>(rg) : q4k_mfma_pick<8, 16>(rg));
    if (64LL * ks * t != n_in) return hipErrorNotSupported;
    hipLaunchKernelGGL(fn, dim3((unsigned)((groups + rg - 1) / rg)), dim3(64 * ks * rg), 0, s, w, x, n_in, n_out,
                       out);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_q4k_gemv(Q4KView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                           float* out, hipStream_t s)
{
    Q4KArgs a{};
    a.qs = w.qs;
    a.dm = w.dm;
    a.sm = w.sm;
    a.out = out;
    a.x = x;
    a.n_in = n_in;
    a.n_out = n_out;
    a.batch = (int)batch;
    a.nch = (int)(n_in / 16);
    const int bt = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
    const int nch64 = a.nch % 64 == 0 ? a.nch / 64 : 0;
    KernelFn fn = nullptr;
    int64_t blocks = 0;
    int threads = 256;
    size_t lds = 0;
    const B1XlShape xsh = b1_xl_shape(nch64, n_out);
    if (bt == 1 && xsh.ks > 0) {
        fn = pick_b1_xl(xsh, nch64);
        threads = 64 * xsh.ks * xsh.g;
        const int64_t rows_per_block = (int64_t)xsh.g * xsh.r;
        blocks = (n_out + rows_per_block - 1) / rows_per_block;
        lds = (size_t)n_in * 4;
    } else if (nch64 > 0 && bt == 1) {
        // 4 rows per wave (a Q4_K chunk costs ~50 VALU operations, so fewer
        // rows per wave than Q8_0; measured best of 2, 4 and 8 on the 8192x3072
        // and 3072x8192 shapes), halved while the grid would hold fewer than
        // 3072 waves
        const B1Shape sh = b1_shape(nch64);
        int r = 4;
        while (r > 1 && (n_out / r) * sh.ks < 3072) r >>= 1;
        fn = r == 4 ? pick_b1_split<4>(nch64) : (r == 2 ? pick_b1_split<2>(nch64) : pick_b1_split<1>(nch64));
        threads = 64 * sh.ks;
        blocks = (n_out + r - 1) / r;
    } else if (nch64 > 0) {
        const int ks = split_ks(nch64);
        const int groups = 4 / ks;
        int r = 4;
        while (r > 1 && n_out / ((int64_t)groups * r) < 512) r >>= 1;
        int r_eff = r;
        switch (bt) {
            case 2:
                fn = r >= 2 ? pick_split<2, 2>(nch64) : pick_split<2, 1>(nch64);
                r_eff = r >= 2 ? 2 : 1;
                break;
            case 4:
                fn = r >= 2 ? pick_split<4, 2>(nch64) : pick_split<4, 1>(nch64);
                r_eff = r >= 2 ? 2 : 1;
                break;
            default:
                fn = pick_split<8, 1>(nch64);
                r_eff = 1;
                break;
        }
        const int64_t rows_per_block = (int64_t)groups * r_eff;
        blocks = (n_out + rows_per_block - 1) / rows_per_block;
    }
    if (!fn) {
        int lpr_log2 = 6;
        while (lpr_log2 > 1 && (1 << lpr_log2) > a.nch) --lpr_log2;
        a.lpr_log2 = lpr_log2;
        switch (bt) {
            case 1: fn = q4k_gemv_general<1>; break;
            case 2: fn = q4k_gemv_general<2>; break;
            case 4: fn = q4k_gemv_general<4>; break;
            default: fn = q4k_gemv_general<8>; break;
        }
        const int64_t rows_per_wave = 64 >> lpr_log2;
        blocks = ((n_out + rows_per_wave - 1) / rows_per_wave + 3) / 4;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), lds, s, a);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
