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
#include "qdec_internal.h"

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

}  // namespace qdec
