// Q6_K dequant-GEMV, its load-time repack and its dequantisation export.
//
// The pages name Q6_K for the embedding and output tensors ("Struct
// QTensorEngine" page: the quantised token embedding path and the output
// projection) and give no byte layout; the one used is the public GGML K-quant
// layout.  A 210-byte super-block holds 256 weights: ql[128] (low four bits of
// the 6-bit quants), qh[64] (high two bits), int8 scales[16], fp16 d.  Weight
// 128h + 32j + l (h = 0, 1; j = 0..3; l = 0..31) takes the low (j < 2) or high
// (j >= 2) nibble of ql[64h + 32(j % 2) + l], bits 2j..2j+1 of qh[32h + l] and
// scale scales[8h + 2j + l / 16]; w = d * scale * (q - 32).
//
// Work unit: a lane takes 16 weights that share their bytes, 128h + 32j + 4m + t
// for j, t = 0..3 (chunk 8h + m of the super-block): one 12-byte load of its
// repacked bits and one 12-byte load of its half-block header (8 scales and d).
// Each weight byte is rebuilt as the signed value 4(q - 32) in one byte -- the
// nibble shifted up two bits, the two high bits with their top bit flipped
// above it -- and converted by one sign-extending conversion, so the products
// with x are exact and nothing cancels; the factor 4 goes into the scale
// (d * scale / 4 is exact).  Per group j: t_j = sum_t 4(q - 32) x, then
// acc += (d * scale_j / 4) * t_j.
//
// Mapping as the Q8_0 and Q4_K kernels: lane j of a wave takes chunks j,
// j + 64, ...; one batch row gives each wave one chunk column (n_in / 1024
// waves per row group, one group per workgroup, 4 rows per wave); other
// batches and widths use a bounds-checked loop over row groups of LPR lanes.
// One batch row at widths 1024, 2048, 3072, 4096, 6144 and 8192 runs instead
// on the integer matrix cores from a second, fragment-tiled copy (see the
// matrix-core section below): x as a fixed-point number per scale group, the
// weights as int8 4(q - 32), about a third of the VALU work per weight.
#include "qdec_internal.h"

#include <algorithm>

namespace qdec {

namespace {

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

struct Q6KArgs {
    const uint8_t* q;
    const uint8_t* hd;
    float* out;
    const float* x;
    int64_t n_in;
    int64_t n_out;
    int batch;
    int lpr_log2;   // general path: lanes per row group
    int nch;        // 16-weight chunks per row = n_in / 16
};

struct Bits12 {
    uint32_t a, b, c;
};

typedef __attribute__((address_space(1))) const uint32_t global_u32;

// 12 bytes as three words from global memory (one dwordx3 load; the explicit
// address space keeps it a global load, whose counter the arithmetic can wait
// on piecewise, rather than a flat one)
__device__ inline Bits12 load12(const uint8_t* base, int64_t off)
{
    const global_u32* w = (const global_u32*)(base + off);
    return Bits12{__builtin_nontemporal_load(w), __builtin_nontemporal_load(w + 1), __builtin_nontemporal_load(w + 2)};
}

// x of chunk c (chunk = 8h + m of super-block c / 16): xv[4j + t] = x[256 sb + 128h + 32j + 4m + t]
__device__ inline void load_xchunk(const float* xrow, int64_t c, float (&xv)[16])
{
    const int64_t sb = c >> 4;
    const int cc = (int)(c & 15);
    const float* base = xrow + sb * 256 + 128 * (cc >> 3) + 4 * (cc & 7);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(base + 32 * j);
        xv[4 * j] = v.x; xv[4 * j + 1] = v.y; xv[4 * j + 2] = v.z; xv[4 * j + 3] = v.w;
    }
}

// The four bytes of group j as signed 4(q - 32): (nibble << 2) | ((hi ^ 2) << 6).
__device__ inline uint32_t group_bytes(const Bits12& q, int j)
{
    const uint32_t lowsrc = (j & 1) ? q.b : q.a;
    const uint32_t nib = ((j < 2) ? lowsrc : (lowsrc >> 4)) & 0x0F0F0F0Fu;
    const uint32_t hi = ((q.c >> (2 * j)) & 0x03030303u) ^ 0x02020202u;
    return (nib << 2) | (hi << 6);
}

// Contribution of one chunk: header words (scales 0..3, scales 4..7, d).
__device__ inline float chunk_dot(const Bits12& q, const Bits12& hd, int m, const float (&xv)[16], float acc)
{
    const float d = fp16_bits_to_f32((uint16_t)(hd.c & 0xffff));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t g = group_bytes(q, j);
        float t = (float)(int8_t)(g & 0xff) * xv[4 * j];
#pragma unroll
        for (int u = 1; u < 4; ++u) t = __builtin_fmaf((float)(int8_t)((g >> (8 * u)) & 0xff), xv[4 * j + u], t);
        // scale byte 2j + (m >= 4) of the half header
        const int sidx = 2 * j + (m >> 2);
        const uint32_t sw = sidx < 4 ? hd.a : hd.b;
        const float sc = (float)(int8_t)((sw >> (8 * (sidx & 3))) & 0xff);
        acc = __builtin_fmaf(d * sc * 0.25f, t, acc);
    }
    return acc;
}

template <int CTRL>
__device__ inline float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

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

// One batch row, n_in a multiple of 1024: KS = n_in / 1024 waves per row group
// (one chunk column each), one group of R rows per workgroup.
template <int R, int KS>
__global__ __launch_bounds__(64 * KS) void q6k_gemv_b1(Q6KArgs a)
{
    __shared__ float part[KS][R];
    const int lane = threadIdx.x & 63;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = (int64_t)blockIdx.x * R;
    const int64_t nsb = a.n_in >> 8;
    const int64_t c = lane + 64 * ks;                  // chunk within the row
    const int64_t sbr = c >> 4;                        // super-block within the row
    const int cc = (int)(c & 15);

    float xv[16];
    load_xchunk(a.x, c, xv);
    // row bases are scalar, the lane's offset within a row is 32-bit
    const int loff_q = (int)(sbr * 192 + cc * 12), loff_h = (int)(sbr * 24 + (cc >> 3) * 12);
    const uint8_t* qrow[R];
    const uint8_t* hrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t rr = row0 + r < a.n_out ? row0 + r : a.n_out - 1;   // keep loads in bounds
        qrow[r] = a.q + rr * nsb * 192;
        hrow[r] = a.hd + rr * nsb * 24;
    }
    Bits12 hv[R], qv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) hv[r] = load12(hrow[r], loff_h);
#pragma unroll
    for (int r = 0; r < R; ++r) qv[r] = load12(qrow[r], loff_q);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(chunk_dot(qv[r], hv[r], cc & 7, xv, 0.0f));

    float v = 0.0f;
    if constexpr (KS > 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) part[ks][r] = acc[r];
        }
        __syncthreads();
        if (ks != 0) return;
        if (lane < R) {
#pragma unroll
            for (int k = 0; k < KS; ++k) v += part[k][lane];
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane == r) v = acc[r];
    }
    if (lane < R && row0 + lane < a.n_out) a.out[row0 + lane] = v;
}

// General path: row groups of LPR lanes, one row per group, bounds-checked loop.
template <int B>
__global__ __launch_bounds__(256) void q6k_gemv_general(Q6KArgs a)
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
    const float* xrow[B];
#pragma unroll
    for (int b = 0; b < B; ++b) xrow[b] = a.x + (int64_t)(b < a.batch ? b : a.batch - 1) * a.n_in;
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    for (int64_t c = j; c < a.nch; c += lpr) {
        const int64_t sbr = c >> 4;
        const int cc = (int)(c & 15);
        const Bits12 qv = load12(a.q, (rr * nsb + sbr) * 192 + cc * 12);
        const Bits12 hv = load12(a.hd, (rr * nsb + sbr) * 24 + (cc >> 3) * 12);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float xv[16];
            load_xchunk(xrow[b], c, xv);
            acc[b] = chunk_dot(qv, hv, cc & 7, xv, acc[b]);
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

// Repack: one thread per super-block (105 halfwords of the GGML block).
__global__ __launch_bounds__(256) void repack_q6k_kernel(const uint16_t* __restrict__ raw, int64_t nblocks,
                                                         uint32_t* __restrict__ qp, uint32_t* __restrict__ hp)
{
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    const uint16_t* src = raw + blk * 105;
    // the block's bytes as 52 little-endian words (ql 0..31, qh 32..47, scales 48..51) and d
    auto word = [&](int k) { return (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16); };
    uint32_t* q = qp + blk * 48;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int ch = 8 * h + m;
            q[3 * ch + 0] = word(16 * h + m);          // ql[64h + 4m ..]
            q[3 * ch + 1] = word(16 * h + 8 + m);      // ql[64h + 32 + 4m ..]
            q[3 * ch + 2] = word(32 + 8 * h + m);      // qh[32h + 4m ..]
        }
    }
    const uint32_t d = src[104];
    uint32_t* hd = hp + blk * 6;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        hd[3 * h + 0] = word(48 + 2 * h);
        hd[3 * h + 1] = word(49 + 2 * h);
        hd[3 * h + 2] = d;
    }
}

// Dequantisation export: one thread per chunk (16 weights); exact in f32.
__global__ __launch_bounds__(256) void dequant_q6k_kernel(Q6KView w, int64_t nchunks, float* __restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= nchunks) return;
    const int64_t sbg = c >> 4;
    const int cc = (int)(c & 15);
    const int h = cc >> 3, m = cc & 7;
    const uint32_t* q = reinterpret_cast<const uint32_t*>(w.q) + c * 3;
    const uint32_t* hd = reinterpret_cast<const uint32_t*>(w.h) + (sbg * 2 + h) * 3;
    const Bits12 qv{q[0], q[1], q[2]};
    const float d = fp16_bits_to_f32((uint16_t)(hd[2] & 0xffff));
    float* o = out + sbg * 256 + 128 * h + 4 * m;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t g = group_bytes(qv, j);
        const int sidx = 2 * j + (m >> 2);
        const float sc = (float)(int8_t)(((sidx < 4 ? hd[0] : hd[1]) >> (8 * (sidx & 3))) & 0xff);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            o[32 * j + t] = d * sc * (0.25f * (float)(int8_t)((g >> (8 * t)) & 0xff));
    }
}

// Tiled repack (the matrix-core GEMV's copy): one thread per 12-byte cell,
// i.e. per (row group G, chunk c, lane l): row 16G + l%16, scale group
// 4(c%4) + l/16 of super-block c/4.  Threads of the first chunk of a
// super-block also write their scale word, and lanes 0..15 of them the d
// halfword.  Rows past n_out are written as zeros.
__global__ __launch_bounds__(256) void repack_q6k_tiled_kernel(const uint8_t* __restrict__ raw, int64_t n_out,
                                                               int64_t nsb, int64_t ncells,
                                                               uint32_t* __restrict__ qt,
                                                               uint32_t* __restrict__ sct,
                                                               uint16_t* __restrict__ dt)
{
    const int64_t cell = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (cell >= ncells) return;
    const int l = (int)(cell & 63);
    const int64_t tile = cell >> 6;            // G * nch + c
    const int64_t nch = nsb * 4;
    const int64_t G = tile / nch;
    const int64_t c = tile % nch;
    const int64_t sb = c >> 2;
    const int cs = (int)(c & 3), g = l >> 4;
    const int64_t row = G * 16 + (l & 15);
    uint32_t n0 = 0, n1 = 0, hw = 0, scw = 0;
    uint16_t d = 0;
    if (row < n_out) {
        const uint8_t* blk = raw + (row * nsb + sb) * 210;
        // weight p = 64 cs + 16 g + b of the super-block: half h = p / 128,
        // quarter j = (p % 128) / 32, position p % 32 = 16 (g % 2) + b
        const int h = cs >> 1, j = 2 * (cs & 1) + (g >> 1);
        const uint8_t* ql = blk + 64 * h + 32 * (j & 1) + 16 * (g & 1);
        const uint8_t* qh = blk + 128 + 32 * h + 16 * (g & 1);
        for (int b = 0; b < 16; ++b) {
            const uint32_t nib = (j < 2 ? ql[b] : (uint32_t)(ql[b] >> 4)) & 15u;
            const uint32_t hi = ((uint32_t)(qh[b] >> (2 * j)) & 3u) ^ 2u;
            const int i = b & 3, t = b >> 2;
            if (t < 2) n0 |= nib << (8 * i + 4 * t);
            else n1 |= nib << (8 * i + 4 * (t - 2));
            hw |= hi << (8 * i + 2 * t);
        }
        if (cs == 0) {
            const uint8_t* sc = blk + 192;
            for (int k = 0; k < 4; ++k) scw |= (uint32_t)sc[4 * k + g] << (8 * k);
            d = (uint16_t)(blk[208] | (blk[209] << 8));
        }
    }
    qt[cell * 3 + 0] = n0;
    qt[cell * 3 + 1] = n1;
    qt[cell * 3 + 2] = hw;
    if (cs == 0) {
        const int64_t st = G * nsb + sb;
        sct[st * 64 + l] = scw;
        if (l < 16) dt[st * 16 + l] = d;
    }
}

// ------------------------------------------------------ matrix cores --
// One batch row on the integer matrix cores, from the tiled copy.  A 768-byte
// tile is 16 rows x one 64-weight chunk (four 16-weight scale groups) and one
// K = 64 step of v_mfma_i32_16x16x64_i8.  Lane l (row n = l % 16, k-group
// g = l / 16) holds scale group g of row n: its 16 B operand bytes are that
// group's weights, each rebuilt as the int8 value 4(q - 32) -- the nibble
// shifted up two bits, the high bit pair (stored with its top bit flipped)
// above it -- by three or four operations per four bytes.
// x is a fixed-point number per scale group s of 16 values:
// X_k = trunc(x_k * 2^(30 - e_s)), |x_k| < 2^e_s over the group, so |X_k| <
// 2^30 and x_k = X_k 2^(e_s - 30) + eps_k, |eps_k| < 2^(e_s - 30).  X_k has
// the signed base-256 digits a_0..a_3 (a_3 within -64..64).  The A operand's
// row 4s + j holds digit j of group s on k-group s and zeros on the other
// three, so the product's row 4s + j, column n, is D_j = sum_k 4(q_k - 32)
// a_j,k over group s of row n: lane l receives in D[0..3] the four digit sums
// of group l / 16 of row l % 16 (the group its own B bytes held), forms
// u = (256 D3 + D2) 2^16 + (256 D1 + D0) and accumulates
//     (d sc) * 2^(e_s - 32) * u,
// d sc exact (11 x 8 significant bits), the power of two exact (the 2 of
// e_s - 32 takes out the factor 4).  Both brackets are multiples of 4; they
// convert exactly while below 2^26 in magnitude, which only an extreme group
// (nearly every quant 0 with digits at the end of their range) can exceed;
// the fma rounds once.  In LDS the A operand is kept as its non-zero part:
// per chunk 16 cells of 16 bytes (group s, digit j), then one zero cell that
// the lanes off the diagonal read.
// A workgroup is RG 16-row groups, each with K split over KS waves of T
// chunks (T % 4 == 0: a wave starts on a super-block).  Each thread loads its
// quads of x and waits for them, then issues every weight load of its wave
// (T tiles; per super-block the scale words and d); while those are in
// flight the workgroup writes the A cells and per scale group e_s - 32.
// Error per output, beyond the f32 rounding of the VALU kernel: at most
// 2^(e_s - 30) <= 2^-29 max_s |x| per x value, times |d sc (q_k - 32)|.
template <int KS, int T, int RG>
__global__ __launch_bounds__(64 * KS * RG) void q6k_gemv_mfma(Q6KTView w, const float* __restrict__ x,
                                                              int64_t n_in, int64_t n_out, float* __restrict__ out)
{
    static_assert(T % 4 == 0 && T >= 4 && T <= 16 && KS * RG <= 16, "T chunks per wave, KS * RG waves");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const uint16_t global_u16;
    constexpr int n = 64 * T * KS;     // n_in
    constexpr int NCH = n / 64;
    constexpr int NW = KS * RG;
    constexpr int NT = 64 * NW;        // threads
    constexpr int NQ = n / 4;          // quads of x
    constexpr int QK = (NQ + NT - 1) / NT;
    constexpr int CB = 272;            // LDS bytes a chunk: 16 A cells, one zero cell
    static_assert(QK <= 4, "quads per thread");
    __shared__ __attribute__((aligned(16))) uint8_t lds[CB * NCH];
    __shared__ __attribute__((aligned(16))) int xe[4][NCH];   // e_s - 32 of group s of chunk c
    __shared__ int wbad[NW];
    __shared__ float red[RG][KS][16];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wv / KS, kw = wv % KS;
    const int64_t groups = q6kt_groups(n_out);
    const int64_t Gw = (int64_t)blockIdx.x * RG + rg;          // this wave's row group
    const int64_t G = Gw < groups ? Gw : groups - 1;           // a spare wave reads the last one
    const int64_t nsb = n_in >> 8;
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
    // every weight load of this wave: T cells of 12 bytes, per super-block
    // the scale word and d of the lane's row
    Bits12 qv[T];
    uint32_t scv[T / 4];
    uint16_t dv[T / 4];
    {
        const int64_t cell0 = (G * NCH + c0) * 64 + lane;
        const uint8_t* qb = w.q + cell0 * 12;
        const global_u32* st = (const global_u32*)w.sc + (G * nsb + c0 / 4) * 64 + lane;
        const global_u16* dt = (const global_u16*)w.d + (G * nsb + c0 / 4) * 16 + (lane & 15);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            qv[t] = load12(qb, (int64_t)t * 768);
            if (t % 4 == 0) {
                scv[t / 4] = __builtin_nontemporal_load(st + (t / 4) * 64);
                dv[t / 4] = __builtin_nontemporal_load(dt + (t / 4) * 16);
            }
        }
    }
    asm volatile("" ::: "memory");
    // A cells and group exponents: quad i holds values 4i .. 4i + 3 of chunk
    // c = i / 16, scale group s = (i / 4) % 4, at bytes 4 (i % 4) of its cells
    int bad = 0;
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        if (64 * wv + k * NT >= NQ) break;
        const int i = tid + k * NT;
        float v[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
        uint32_t amax = max(max(__builtin_bit_cast(uint32_t, v[0]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[1]) & 0x7fffffffu),
                            max(__builtin_bit_cast(uint32_t, v[2]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[3]) & 0x7fffffffu));
        // over the group's 4 quads (4 consecutive lanes): lane ^ 1, lane ^ 2
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
        const bool fin = amax < 0x7f800000u;
        if (__builtin_amdgcn_ballot_w64(!fin) != 0) {
            // rare: a non-finite group converts zeros (every output is NaN;
            // an infinity or NaN has no defined int conversion)
            bad |= !fin;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fin ? v[e] : 0.0f;
        }
        // amax = m 2^e with 0.5 <= m < 1, so every |x| < 2^e (e = 0 for zeros)
        const int e_s = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, amax));
        // X = trunc(x 2^(30 - e)), |X| < 2^30; its signed base-256 digits are
        // the bytes of X + 0x80808080, each less 0x80
        uint32_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = (uint32_t)(int)__builtin_amdgcn_ldexpf(v[e], 30 - e_s) + 0x80808080u;
        // word j = digit j of the 4 values
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
        const int c = i >> 4, s = (i >> 2) & 3, qq = i & 3;
        uint8_t* cell = lds + CB * c + 64 * s + 4 * qq;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(cell + 16 * j) = wd[j];
        if (qq == 0) xe[s][c] = e_s - 32;
        if ((i & 15) == 0) *reinterpret_cast<uint4*>(lds + CB * c + 256) = make_uint4(0u, 0u, 0u, 0u);
    }
    // a non-finite x makes every output NaN
    const uint64_t badm = __builtin_amdgcn_ballot_w64(bad != 0);
    if (lane == 0) wbad[wv] = badm != 0;
    __syncthreads();
    const bool any_bad = __builtin_amdgcn_ballot_w64(lane < NW && wbad[lane < NW ? lane : 0] != 0) != 0;

    // A operand of lane (row m = lane % 16, k-group g = lane / 16): cell m of
    // the chunk on the diagonal (m / 4 == g), the zero cell elsewhere; the D
    // side and the B bytes of the lane are group g of row lane % 16
    const int m = lane & 15, g = lane >> 4;
    const int aoff = CB * c0 + ((m >> 2) == g ? 16 * m : 256);
    int eb[T];
#pragma unroll
    for (int q = 0; q < T / 4; ++q) {
        const int4 e4 = *reinterpret_cast<const int4*>(&xe[g][c0 + 4 * q]);
        eb[4 * q] = e4.x;
        eb[4 * q + 1] = e4.y;
        eb[4 * q + 2] = e4.z;
        eb[4 * q + 3] = e4.w;
    }
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const i32x4 A = *reinterpret_cast<const i32x4*>(lds + aoff + CB * t);
        const uint32_t n0 = qv[t].a, n1 = qv[t].b, hw = qv[t].c;
        const i32x4 B = {(int)(((n0 << 2) & 0x3C3C3C3Cu) | ((hw << 6) & 0xC0C0C0C0u)),
                         (int)(((n0 >> 2) & 0x3C3C3C3Cu) | ((hw << 4) & 0xC0C0C0C0u)),
                         (int)(((n1 << 2) & 0x3C3C3C3Cu) | ((hw << 2) & 0xC0C0C0C0u)),
                         (int)(((n1 >> 2) & 0x3C3C3C3Cu) | (hw & 0xC0C0C0C0u))};
        const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
        const float u = __builtin_fmaf((float)(D[3] * 256 + D[2]), 65536.0f, (float)(D[1] * 256 + D[0]));
        const float d = fp16_bits_to_f32(dv[t / 4]);
        const float sc = (float)(int8_t)((scv[t / 4] >> (8 * (t % 4))) & 0xffu);
        acc = __builtin_fmaf(d * sc, __builtin_amdgcn_ldexpf(u, eb[t]), acc);
    }
    // row r: its four groups in lanes r + 16 g, then the KS waves of its
    // row group in order
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
    if (any_bad) acc = __builtin_nanf("");
    const int64_t row = Gw * 16 + lane;
    if (lane < 16 && Gw < groups && row < n_out) out[row] = acc;
}

// Two to eight batch rows on the integer matrix cores, from the same tiled
// copy and with the same arithmetic per row as q6k_gemv_mfma: each chunk's B
// operand (the unpacked quants) and d sc are formed once and multiplied by
// every batch row's A cells, one MFMA per row.  The rows' A cells and
// exponents take B x n_in x 4.25 bytes of LDS (B n_in <= 32768, so 8 rows up
// to 4096 columns, 4 up to 8192: at most 139 KB); RG row groups a workgroup
// (2, or 3-4 for tall matrices, see q6k_rows_rg), each with K over KS waves
// of T chunks.  B is the batch rounded up to 2, 4
// or 8: rows past the real batch repeat its last row and are not stored.  A
// non-finite x makes every output of its batch row NaN.
template <int B, int KS, int T, int RG>
__global__ __launch_bounds__(64 * KS * RG) void q6k_gemv_mfma_rows(Q6KTView w, const float* __restrict__ x,
                                                                     int64_t n_in, int64_t n_out, int batch,
                                                                     float* __restrict__ out)
{
    static_assert(T % 4 == 0 && T >= 4 && T <= 16 && KS * RG <= 16, "T chunks per wave, KS * RG waves");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const uint16_t global_u16;
    constexpr int n = 64 * T * KS;     // n_in
    constexpr int NCH = n / 64;
    constexpr int NW = KS * RG;
    constexpr int NT = 64 * NW;
    constexpr int NQ = n / 4;          // quads of one batch row
    constexpr int QK = (B * NQ + NT - 1) / NT;
    constexpr int CB = 272;            // LDS bytes a chunk and row: 16 A cells, one zero cell
    static_assert(QK <= 16 && B * n <= 32768, "quads per thread, LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[B * CB * NCH];
    __shared__ __attribute__((aligned(16))) int xe[B][4][NCH];   // e_s - 32 of row b, group s, chunk c
    __shared__ uint32_t wbad[NW];
    __shared__ float red[RG][KS][B][16];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wv / KS, kw = wv % KS;
    const int64_t groups = q6kt_groups(n_out);
    const int64_t Gw = (int64_t)blockIdx.x * RG + rg;
    const int64_t G = Gw < groups ? Gw : groups - 1;           // a spare wave reads the last group
    const int64_t nsb = n_in >> 8;
    const int c0 = kw * T;

    // quads it = tid + k NT of the B rows: row it / NQ (whole waves, NQ % 64
    // == 0), quad it % NQ
    float4 xv[QK];
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        const int it = tid + k * NT;
        if (64 * wv + k * NT < B * NQ) {
            const int b = it / NQ;
            const int br = b < batch ? b : batch - 1;
            xv[k] = reinterpret_cast<const float4*>(x + (int64_t)br * n_in)[it % NQ];
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    asm volatile("" ::: "memory");
    Bits12 qv[T];
    uint32_t scv[T / 4];
    uint16_t dv[T / 4];
    {
        const int64_t cell0 = (G * NCH + c0) * 64 + lane;
        const uint8_t* qb = w.q + cell0 * 12;
        const global_u32* st = (const global_u32*)w.sc + (G * nsb + c0 / 4) * 64 + lane;
        const global_u16* dt = (const global_u16*)w.d + (G * nsb + c0 / 4) * 16 + (lane & 15);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            qv[t] = load12(qb, (int64_t)t * 768);
            if (t % 4 == 0) {
                scv[t / 4] = __builtin_nontemporal_load(st + (t / 4) * 64);
                dv[t / 4] = __builtin_nontemporal_load(dt + (t / 4) * 16);
            }
        }
    }
    asm volatile("" ::: "memory");
    // A cells and exponents of every row (as in q6k_gemv_mfma, at row offset
    // b NCH CB)
    uint32_t badm = 0;
#pragma unroll
    for (int k = 0; k < QK; ++k) {
        if (64 * wv + k * NT >= B * NQ) break;
        const int it = tid + k * NT;
        const int b = it / NQ, i = it % NQ;
        float v[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
        uint32_t amax = max(max(__builtin_bit_cast(uint32_t, v[0]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[1]) & 0x7fffffffu),
                            max(__builtin_bit_cast(uint32_t, v[2]) & 0x7fffffffu,
                                __builtin_bit_cast(uint32_t, v[3]) & 0x7fffffffu));
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0xB1, 0xF, 0xF, false));
        amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, 0x4E, 0xF, 0xF, false));
        const bool fin = amax < 0x7f800000u;
        if (__builtin_amdgcn_ballot_w64(!fin) != 0) {
            // rare: a non-finite group converts zeros (its row's outputs are NaN)
            badm |= fin ? 0u : 1u << b;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fin ? v[e] : 0.0f;
        }
        const int e_s = __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, amax));
        uint32_t y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = (uint32_t)(int)__builtin_amdgcn_ldexpf(v[e], 30 - e_s) + 0x80808080u;
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
        const int c = i >> 4, sg = (i >> 2) & 3, qq = i & 3;
        uint8_t* chunk = lds + (b * NCH + c) * CB;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(chunk + 64 * sg + 16 * j + 4 * qq) = wd[j];
        if (qq == 0) xe[b][sg][c] = e_s - 32;
        if ((i & 15) == 0) *reinterpret_cast<uint4*>(chunk + 256) = make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t wm = 0;
#pragma unroll
    for (int b = 0; b < B; ++b)
        if (__builtin_amdgcn_ballot_w64(((badm >> b) & 1u) != 0) != 0) wm |= 1u << b;
    if (lane == 0) wbad[wv] = wm;
    __syncthreads();
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) bad |= wbad[k];

    const int m = lane & 15, g = lane >> 4;
    const int aoff = CB * c0 + ((m >> 2) == g ? 16 * m : 256);
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    int4 e4[B];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t % 4 == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b) e4[b] = *reinterpret_cast<const int4*>(&xe[b][g][c0 + t]);
        }
        const uint32_t n0 = qv[t].a, n1 = qv[t].b, hw = qv[t].c;
        const i32x4 Bop = {(int)(((n0 << 2) & 0x3C3C3C3Cu) | ((hw << 6) & 0xC0C0C0C0u)),
                           (int)(((n0 >> 2) & 0x3C3C3C3Cu) | ((hw << 4) & 0xC0C0C0C0u)),
                           (int)(((n1 << 2) & 0x3C3C3C3Cu) | ((hw << 2) & 0xC0C0C0C0u)),
                           (int)(((n1 >> 2) & 0x3C3C3C3Cu) | (hw & 0xC0C0C0C0u))};
        const float dsc = fp16_bits_to_f32(dv[t / 4]) * (float)(int8_t)((scv[t / 4] >> (8 * (t % 4))) & 0xffu);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const i32x4 A = *reinterpret_cast<const i32x4*>(lds + b * NCH * CB + aoff + CB * t);
            const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, Bop, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const float u = __builtin_fmaf((float)(D[3] * 256 + D[2]), 65536.0f, (float)(D[1] * 256 + D[0]));
            const int eb = (t % 4) == 0 ? e4[b].x : (t % 4) == 1 ? e4[b].y : (t % 4) == 2 ? e4[b].z : e4[b].w;
            acc[b] = __builtin_fmaf(dsc, __builtin_amdgcn_ldexpf(u, eb), acc[b]);
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        acc[b] += __shfl_xor(acc[b], 16, 64);
        acc[b] += __shfl_xor(acc[b], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
        for (int b = 0; b < B; ++b) red[rg][kw][b][lane] = acc[b];
    }
    __syncthreads();
    if (kw != 0) return;
    const int64_t row = Gw * 16 + lane;
    if (lane < 16 && Gw < groups && row < n_out) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (b >= batch) break;
            float sm = red[rg][0][b][lane];
#pragma unroll
            for (int k = 1; k < KS; ++k) sm += red[rg][k][b][lane];
            out[(int64_t)b * n_out + row] = (bad >> b) & 1u ? __builtin_nanf("") : sm;
        }
    }
}

// K split: n_in = 64 KS T, T = 8, 12 or 16 chunks a wave: 1024 on 2 waves,
// 2048 .. 4096 on 4, 6144 and 8192 on 8.
bool q6k_mfma_shape(int64_t n_in, int* ks, int* t)
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

// Row groups a workgroup: two from 512 groups on (sharing the x operands),
// within 16 waves a workgroup.
int q6k_mfma_rg(int64_t groups, int ks) { return groups >= 512 && 2 * ks <= 16 ? 2 : 1; }

using KernelFnT6 = void (*)(Q6KTView, const float*, int64_t, int64_t, float*);

template <int KS, int T>
KernelFnT6 q6k_mfma_pick(int rg)
{
    return rg == 2 ? q6k_gemv_mfma<KS, T, 2> : q6k_gemv_mfma<KS, T, 1>;
}

using KernelFnR6 = void (*)(Q6KTView, const float*, int64_t, int64_t, int, float*);

// Rows rounded up to 2, 4 or 8, within B n_in <= 32768.
int q6k_rows_b(int64_t n_in, int64_t batch)
{
    const int b = batch <= 2 ? 2 : batch <= 4 ? 4 : 8;
    return b * n_in <= 32768 ? b : 0;
}

// 5..8 rows at 6144 and 8192 columns (beyond one workgroup's LDS) run as two
// launches of (batch + 1) / 2 and the remaining rows on x and out offset by
// the first part's rows.
bool q6k_rows_split(int64_t n_in, int64_t batch)
{
    return batch > 4 && batch <= 8 && !q6k_rows_b(n_in, batch) && q6k_rows_b(n_in, 4);
}

// Row groups a workgroup of the multi-row kernel: 3 for 4 and 8 rows of a
// tall matrix (>= 2048 row groups, so >= 680 workgroups remain), which cuts
// the x preparation per weight row by a third against 2.  Measured at
// 128256 x 3072 (graph-replayed): b4 84.2 -> 76.8 us, b8 189 -> 151-153 us;
// 4 row groups were slower at b4 (93.9) and spill at b8.  Below 512 row
// groups one (as the one-row kernel), so that a 3072-row matrix still has
// 192 workgroups, where the x quads still fit the threads (B T / 4 <= 16);
// else 2.
int q6k_rows_rg(int64_t groups, int ks, int t, int b)
{
    if (groups < 512 && b * t <= 64) return 1;
    if (ks > 4 || groups < 2048) return 2;
    return b >= 4 ? 3 : 2;
}

template <int KS, int T>
KernelFnR6 q6k_rows_pick_rg(int b, int rg)
{
    if constexpr (8 * 64 * KS * T <= 32768) {
        if constexpr (3 * KS <= 16) {
            if (b == 8 && rg == 3) return q6k_gemv_mfma_rows<8, KS, T, 3>;
        }
        if constexpr (8 * T <= 64) {
            if (b == 8 && rg == 1) return q6k_gemv_mfma_rows<8, KS, T, 1>;
        }
        if (b == 8) return rg == 2 ? q6k_gemv_mfma_rows<8, KS, T, 2> : nullptr;
    }
    if constexpr (4 * 64 * KS * T <= 32768) {
        if constexpr (3 * KS <= 16) {
            if (b == 4 && rg == 3) return q6k_gemv_mfma_rows<4, KS, T, 3>;
        }
        if (b == 4 && rg == 1) return q6k_gemv_mfma_rows<4, KS, T, 1>;
        if (b == 4) return rg == 2 ? q6k_gemv_mfma_rows<4, KS, T, 2> : nullptr;
    }
    if (b != 2) return nullptr;
    return rg == 2 ? q6k_gemv_mfma_rows<2, KS, T, 2> : rg == 1 ? q6k_gemv_mfma_rows<2, KS, T, 1> : nullptr;
}

KernelFnR6 q6k_rows_pick(int ks, int t, int b, int rg)
{
    switch (ks * 100 + t) {
        case 208: return q6k_rows_pick_rg<2, 8>(b, rg);
        case 408: return q6k_rows_pick_rg<4, 8>(b, rg);
        case 412: return q6k_rows_pick_rg<4, 12>(b, rg);
        case 416: return q6k_rows_pick_rg<4, 16>(b, rg);
        case 812: return rg <= 2 ? q6k_rows_pick_rg<8, 12>(b, rg) : nullptr;
        case 816: return rg <= 2 ? q6k_rows_pick_rg<8, 16>(b, rg) : nullptr;
        default: return nullptr;
    }
}

using KernelFn = void (*)(Q6KArgs);

template <int R>
KernelFn pick_b1(int nch64)
{
    switch (nch64) {
        case 1: return q6k_gemv_b1<R, 1>;
        case 2: return q6k_gemv_b1<R, 2>;
        case 3: return q6k_gemv_b1<R, 3>;
        case 4: return q6k_gemv_b1<R, 4>;
        case 6: return q6k_gemv_b1<R, 6>;
        case 8: return q6k_gemv_b1<R, 8>;
        default: return nullptr;
    }
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_repack_q6k(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s)
{
    const Q6KView v = q6k_view(dst, n_in, n_out);
    const int64_t nblocks = (n_in / 256) * n_out;
    hipLaunchKernelGGL(repack_q6k_kernel, dim3(grid_for(nblocks, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(raw), nblocks,
                       reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(v.q)),
                       reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(v.h)));
    count_launch();
    return hipGetLastError();
}

hipError_t launch_dequant_q6k(Q6KView w, int64_t n_in, int64_t n_out, float* out, hipStream_t s)
{
    const int64_t nchunks = n_out * n_in / 16;
    hipLaunchKernelGGL(dequant_q6k_kernel, dim3(grid_for(nchunks, 256)), dim3(256), 0, s, w, nchunks, out);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_q6k_gemv(Q6KView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                           hipStream_t s)
{
    Q6KArgs a{};
    a.q = w.q;
    a.hd = w.h;
    a.out = out;
    a.x = x;
    a.n_in = n_in;
    a.n_out = n_out;
    a.batch = (int)batch;
    a.nch = (int)(n_in / 16);
    const int nch64 = a.nch % 64 == 0 ? a.nch / 64 : 0;
    KernelFn fn = nullptr;
    int64_t blocks = 0;
    int threads = 256;
    if (batch == 1 && nch64 > 0) {
        // 4 rows per wave, halved while the grid would hold fewer than 3072 waves
        int r = 4;
        while (r > 1 && (n_out / r) * nch64 < 3072) r >>= 1;
        fn = r == 4 ? pick_b1<4>(nch64) : (r == 2 ? pick_b1<2>(nch64) : pick_b1<1>(nch64));
        threads = 64 * nch64;
        blocks = (n_out + r - 1) / r;
    }
    if (!fn) {
        int lpr_log2 = 6;
        while (lpr_log2 > 1 && (1 << lpr_log2) > a.nch) --lpr_log2;
        a.lpr_log2 = lpr_log2;
        const int bt = a.batch <= 1 ? 1 : a.batch <= 2 ? 2 : a.batch <= 4 ? 4 : 8;
        switch (bt) {
            case 1: fn = q6k_gemv_general<1>; break;
            case 2: fn = q6k_gemv_general<2>; break;
            case 4: fn = q6k_gemv_general<4>; break;
            default: fn = q6k_gemv_general<8>; break;
        }
        const int64_t rows_per_wave = 64 >> lpr_log2;
        blocks = ((n_out + rows_per_wave - 1) / rows_per_wave + 3) / 4;
        threads = 256;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(threads), 0, s, a);
    count_launch();
    return hipGetLastError();
}

hipError_t launch_repack_q6k_tiled(const uint8_t* raw, int64_t n_in, int64_t n_out, void* dst, hipStream_t s)
{
    const Q6KTView v = q6kt_view(dst, n_in, n_out);
    const int64_t nsb = n_in / 256, ncells = q6kt_groups(n_out) * (n_in / 64) * 64;
    hipLaunchKernelGGL(repack_q6k_tiled_kernel, dim3(grid_for(ncells, 256)), dim3(256), 0, s, raw, n_out, nsb,
                       ncells, reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(v.q)),
                       const_cast<uint32_t*>(v.sc), const_cast<uint16_t*>(v.d));
    count_launch();
    return hipGetLastError();
}

bool q6k_mfma_supported(int64_t n_in, int64_t batch)
{
    int ks = 0, t = 0;
    if (batch < 1 || batch > 8 || !q6k_mfma_shape(n_in, &ks, &t)) return false;
    return batch == 1 || q6k_rows_b(n_in, batch) > 0 || q6k_rows_split(n_in, batch);
}

std::string q6k_mfma_plan_check(int64_t n_in, int64_t n_out, int64_t batch)
{
    if (q6k_rows_split(n_in, batch)) {
        const int64_t b0 = (batch + 1) / 2;
        const std::string e = q6k_mfma_plan_check(n_in, n_out, b0);
        return e.empty() ? q6k_mfma_plan_check(n_in, n_out, batch - b0) : e;
    }
    int ks = 0, t = 0;
    if (!q6k_mfma_shape(n_in, &ks, &t)) return "q6k matrix-core GEMV: unsupported width " + std::to_string(n_in);
    if (64LL * ks * t != n_in) return "q6k matrix-core GEMV: K split does not cover the row";
    if (batch > 1 && !q6k_rows_b(n_in, batch)) return "q6k matrix-core GEMV: batch rows x width beyond LDS";
    const int64_t groups = q6kt_groups(n_out), nch = n_in / 64, nsb = n_in / 256;
    const int rg = batch > 1 ? q6k_rows_rg(groups, ks, t, q6k_rows_b(n_in, batch)) : q6k_mfma_rg(groups, ks);
    const int64_t grid = (groups + rg - 1) / rg;
    if (grid <= 0 || grid > 0x7fffffffLL) return "q6k matrix-core GEMV: grid out of range";
    // the last wave reads row group min(grid rg - 1, groups - 1), chunks up to
    // (ks - 1) t + t - 1 = nch - 1, super-blocks up to nsb - 1
    const int64_t g_last = std::min<int64_t>(grid * rg - 1, groups - 1);
    const int64_t q_end = ((g_last * nch + (int64_t)(ks - 1) * t + t - 1) * 64 + 63) * 12 + 12;
    const int64_t sc_end = ((g_last * nsb + nsb - 1) * 64 + 63) * 4 + 4;
    const int64_t d_end = ((g_last * nsb + nsb - 1) * 16 + 15) * 2 + 2;
    const int64_t g = groups;
    if (q_end > g * nch * 768 || sc_end > g * nsb * 256 || d_end > g * nsb * 32)
        return "q6k matrix-core GEMV: a weight read runs past the tiled copy";
    // x: quads tid + k NT below B n / 4, rows past the batch reading its last
    // row; out: rows below n_out and batch rows below batch (in the kernel)
    const int64_t nt = 64LL * ks * rg, nq = n_in / 4, bp = batch > 1 ? q6k_rows_b(n_in, batch) : 1;
    if (nq % 64 != 0 || (bp * nq + nt - 1) / nt > (batch > 1 ? 16 : 4))
        return "q6k matrix-core GEMV: x quads do not fit the threads";
    return "";
}

hipError_t launch_q6k_gemv_mfma(Q6KTView w, int64_t n_in, int64_t n_out, int64_t batch, const float* x, float* out,
                                hipStream_t s)
{
    int ks = 0, t = 0;
    if (!q6k_mfma_shape(n_in, &ks, &t) || !q6k_mfma_plan_check(n_in, n_out, batch).empty())
        return hipErrorInvalidConfiguration;
    if (q6k_rows_split(n_in, batch)) {
        const int64_t b0 = (batch + 1) / 2;
        const hipError_t e = launch_q6k_gemv_mfma(w, n_in, n_out, b0, x, out, s);
        if (e != hipSuccess) return e;
        return launch_q6k_gemv_mfma(w, n_in, n_out, batch - b0, x + b0 * n_in, out + b0 * n_out, s);
    }
    const int64_t groups = q6kt_groups(n_out);
    if (batch > 1) {
        const int b = q6k_rows_b(n_in, batch), rg = q6k_rows_rg(groups, ks, t, b);
        const KernelFnR6 fr = q6k_rows_pick(ks, t, b, rg);
        if (!fr) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(fr, dim3((unsigned)((groups + rg - 1) / rg)), dim3(64 * ks * rg), 0, s, w, x, n_in, n_out,
                           (int)batch, out);
        count_launch();
        return hipGetLastError();
    }
    const int rg = q6k_mfma_rg(groups, ks);
    KernelFnT6 fn = ks == 2 ? q6k_mfma_pick<2, 8>(rg)
                  : ks == 4 ? (t == 8 ? q6k_mfma_pick<4, 8>(rg) : t == 12 ? q6k_mfma_pick<4, 12>(rg)
                                                                          : q6k_mfma_pick<4, 16>(rg))
                            : (t == 12 ? q6k_mfma_pick<8, 12>(rg) : q6k_mfma_pick<8, 16>(rg));
    hipLaunchKernelGGL(fn, dim3((unsigned)((groups + rg - 1) / rg)), dim3(64 * ks * rg), 0, s, w, x, n_in, n_out,
                       out);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
