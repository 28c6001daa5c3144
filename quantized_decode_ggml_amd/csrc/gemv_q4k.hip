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

}  // namespace

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
