// Batched prefill-shaped GEMM on gfx950 MFMA.
//
// What is computed (rustdoc source view of weight_cache.rs, try_cuda_batch_gemv
// and its doc comment): for each of `batch` packed rows of hidden (n_in wide),
// out[b][i] = sum_j W[i][j] * x[b][j], i.e. C[m x n] = A[m x k] * B[k x n] with
// m = batch, k = n_in, n = n_out and B = W transposed.  That page pads every
// dimension to a multiple of 16 with zeros and trims the result; here the tile
// loads zero-fill past the edges and the stores are predicated, which is the
// same product.
//
// Precision: both operands are rounded to bf16 (round to nearest even) and
// contracted on v_mfma_f32_16x16x32_bf16 with f32 accumulation.  The Q8_0
// weight is first dequantised exactly in f32 (d*q), then rounded.  The pages
// record that f16 tensor-core operands gave unusable results on their
// single-token path; bf16 keeps the f32 exponent range, and the error per
// product is at most about 2*2^-9 relative.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C over a slice
// of K; each of its four waves computes 64 x 64 with 4 x 4 MFMA 16x16x32
// tiles.  K advances 64 at a time (two Q8_0 blocks).  Both operands are staged
// in LDS as bf16 rows (K contiguous, padded by 8 elements against bank
// conflicts), double-buffered: the global loads of step k+1 are in flight
// while step k runs on MFMA.
//
// Parallelism: with few output tiles (the prefill batch is 128 or 512 rows) K
// is split into S slices so that the grid has at least one workgroup per CU;
// the slices add their partial tiles into the output with fire-and-forget f32
// atomics (a fill kernel zeroes the output first).  Each atomic costs far more
// than a store, so S stays at the smallest value that fills the CUs.  Block
// ids go to the XCDs round-robin, which spreads the m-tiles that share a
// weight tile over all L2s (measured faster than grouping consecutive tiles
// on one XCD).
#include "qdec_internal.h"

namespace qdec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride in bf16 elements (144 bytes)

struct GemmArgs {
    const float* x;        // M x K f32
    const int8_t* q;       // Q8_0 q plane (N x K) or nullptr
    const uint16_t* d;     // Q8_0 d plane (N x K/32)
    const float* wf;       // dense f32 W (N x K) or nullptr
    float* out;            // M x N f32
    int64_t M, N, K;
    int64_t mtiles, ntiles;
    int64_t kslice;        // K per split (multiple of BK)
    int splits;
};

__device__ inline float fp16_bits_to_f32(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, sizeof v);
    return static_cast<float>(v);
}

__device__ inline bf16x4 to_bf16x4(float4 v)
{
    bf16x4 r;
    r[0] = (__bf16)v.x;
    r[1] = (__bf16)v.y;
    r[2] = (__bf16)v.z;
    r[3] = (__bf16)v.w;
    return r;
}

// Global -> register staging of one 128 x 64 f32 tile (rows r0.., cols k0..):
// 2048 float4, 8 per thread, consecutive threads on consecutive float4s.
__device__ inline void load_f32_tile(const float* __restrict__ src, int64_t rows, int64_t K,
                                     int64_t kend, int64_t r0, int64_t k0, float4 (&reg)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx >> 4, c4 = idx & 15;
        const int64_t gr = r0 + row, gk = k0 + c4 * 4;
        reg[i] = (gr < rows && gk < kend) ? *reinterpret_cast<const float4*>(src + gr * K + gk)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__device__ inline void store_f32_tile(__bf16* lds, const float4 (&reg)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx >> 4, c4 = idx & 15;
        *reinterpret_cast<bf16x4*>(lds + row * LDK + c4 * 4) = to_bf16x4(reg[i]);
    }
}

// Q8_0 weight tile: 128 rows x 64 q bytes; thread t takes row t/2, block t%2
// (32 weights = two 16-byte loads) and that block's fp16 scale.
struct QTileReg {
    uint4 q0, q1;
    uint16_t d;
};

__device__ inline void load_q8_tile(const GemmArgs& a, int64_t kend, int64_t n0, int64_t k0, QTileReg& reg)
{
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int64_t gn = n0 + row, gk = k0 + half * 32;
    if (gn < a.N && gk < kend) {
        const uint4* p = reinterpret_cast<const uint4*>(a.q + gn * a.K + gk);
        reg.q0 = p[0];
        reg.q1 = p[1];
        reg.d = a.d[gn * (a.K >> 5) + (gk >> 5)];
    } else {
        reg.q0 = make_uint4(0, 0, 0, 0);
        reg.q1 = reg.q0;
        reg.d = 0;
    }
}

__device__ inline void store_q8_tile(__bf16* lds, const QTileReg& reg)
{
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
    const float d = fp16_bits_to_f32(reg.d);
    const uint32_t w[8] = {reg.q0.x, reg.q0.y, reg.q0.z, reg.q0.w, reg.q1.x, reg.q1.y, reg.q1.z, reg.q1.w};
    __bf16* dst = lds + row * LDK + half * 32;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bf16x8 v;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t word = w[2 * k + (t >> 2)];
            v[t] = (__bf16)(d * (float)(int8_t)((word >> (8 * (t & 3))) & 0xff));
        }
        *reinterpret_cast<bf16x8*>(dst + 8 * k) = v;
    }
}

template <bool QUANT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a)
{
    __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * LDK];

    // block id -> (k slice, n tile, m tile), k fastest
    const int64_t id = blockIdx.x;
    const int64_t slice = id % a.splits;
    const int64_t tile = id / a.splits;
    const int64_t n0 = (tile % a.ntiles) * BN;
    const int64_t m0 = (tile / a.ntiles) * BM;
    const int64_t kbeg = slice * a.kslice;
    const int64_t kend = kbeg + a.kslice < a.K ? kbeg + a.kslice : a.K;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    float4 xr[8];
    float4 wr[8];
    QTileReg qr;
    const int64_t nk = (kend - kbeg + BK - 1) / BK;

    load_f32_tile(a.x, a.M, a.K, kend, m0, kbeg, xr);
    if (QUANT) load_q8_tile(a, kend, n0, kbeg, qr);
    else load_f32_tile(a.wf, a.N, a.K, kend, n0, kbeg, wr);
    store_f32_tile(As[0], xr);
    if (QUANT) store_q8_tile(Bs[0], qr);
    else store_f32_tile(Bs[0], wr);
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k0 = kbeg + (kt + 1) * BK;
            load_f32_tile(a.x, a.M, a.K, kend, m0, k0, xr);
            if (QUANT) load_q8_tile(a, kend, n0, k0, qr);
            else load_f32_tile(a.wf, a.N, a.K, kend, n0, k0, wr);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[4], bfr[4];
            const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + i * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            store_f32_tile(As[cur ^ 1], xr);
            if (QUANT) store_q8_tile(Bs[cur ^ 1], qr);
            else store_f32_tile(Bs[cur ^ 1], wr);
        }
        __syncthreads();
    }

    // D layout of the 16x16 MFMA: lane holds column (lane % 16) and rows
    // 4*(lane / 16) + 0..3.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
                if (m >= a.M) continue;
                if (a.splits == 1) a.out[m * a.N + n] = acc[i][j][e];
                else unsafeAtomicAdd(a.out + m * a.N + n, acc[i][j][e]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, int64_t n4, float* __restrict__ tail,
                                                   int64_t ntail)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < ntail) tail[t] = 0.f;
}

// Grid plan: K slices so that tiles * slices reaches 256 workgroups (one per
// CU), each slice at least 512 deep (8 K steps) and a multiple of BK.
GemmArgs plan(int64_t M, int64_t N, int64_t K)
{
    GemmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.mtiles = (M + BM - 1) / BM;
    a.ntiles = (N + BN - 1) / BN;
    const int64_t tiles = a.mtiles * a.ntiles;
    int splits = 1;
    while (tiles * splits < 256 && K / (splits * 2) >= 512) splits *= 2;
    a.kslice = ((K + splits - 1) / splits + BK - 1) / BK * BK;
    a.splits = (int)((K + a.kslice - 1) / a.kslice);
    return a;
}

hipError_t launch(GemmArgs& a, bool quant, hipStream_t s)
{
    if (a.splits > 1) {
        const int64_t n = a.M * a.N;
        const int64_t n4 = n / 4;
        const int64_t ntail = n - n4 * 4;
        int64_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<float4*>(a.out), n4, a.out + n4 * 4, ntail);
        count_launch();
    }
    const dim3 grid((unsigned)(a.mtiles * a.ntiles * a.splits));
    if (quant) hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, dim3(256), 0, s, a);
    count_launch();
    return hipGetLastError();
}

}  // namespace

hipError_t launch_q8_0_gemm(Q8View w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                            float* out, hipStream_t s)
{
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.q = w.q;
    a.d = w.d;
    a.out = out;
    return launch(a, true, s);
}

hipError_t launch_f32_gemm(const float* wf, int64_t n_in, int64_t n_out, int64_t batch,
                           const float* x, float* out, hipStream_t s)
{
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.wf = wf;
    a.out = out;
    return launch(a, false, s);
}

}  // namespace qdec
