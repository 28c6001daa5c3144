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
// Two kernels:
//  - gemm_dma (Q8_0 weights, K % 64 == 0, even N, with a workspace): every
//    operand streamed into LDS by DMA, eight waves per workgroup, B fragments
//    dequantised in registers (described at the kernel).  With few output
//    tiles K is split into slices whose partial products a small kernel sums
//    in slice order.
//    The same kernel also reads the bf16 copy of a dense f32 weight (made by
//    qdec_prepare) the way it reads x: nothing to dequantise, K % 64 == 0.
//  - gemm_bf16_kernel (dense f32 weights without that copy, and Q8_0 shapes
//    off the DMA path or without a workspace): a 256-thread workgroup computes a 128 x 128 tile of
//    C over a slice of K, four waves of 64 x 64 with 4 x 4 MFMA 16x16x32 tiles;
//    both operands register-staged into LDS as bf16 rows (K contiguous, padded
//    by 8 elements against bank conflicts), double-buffered.  Its K slices
//    write partial products to the workspace when there is one, else add them
//    into a zeroed output with f32 atomics.
// Block ids go to the XCDs round-robin; with the tile index n-fastest the m
// tiles that share a weight tile land on one XCD whenever the n-tile count is
// a multiple of 8.
#include <cstdio>
#include <string>

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
    float* part;           // splits > 1: slice s writes part[s][M][N] (workspace), or null: atomics into a zeroed out
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
                else if (a.part) a.part[(slice * a.M + m) * a.N + n] = acc[i][j][e];
                else unsafeAtomicAdd(a.out + m * a.N + n, acc[i][j][e]);
            }
        }
    }
}

// ------------------------------------------------------------ DMA-fed --
// Q8_0 GEMM with every operand streamed global -> LDS by DMA
// (global_load_lds), for K % 64 == 0 and even N.  A 512-thread workgroup
// (eight waves, two per SIMD) computes a 128 x 128 tile of C over a K slice:
// wave w takes k-half w/4 of every 64-k stage and the 128 x 32 block of
// output columns 32*(w%4), i.e. 8 x 2 MFMA 16x16x32 tiles whose B fragments
// it dequantises itself from the int8 bytes in LDS (each weight is
// dequantised once per workgroup; nothing is written back to LDS).  The two
// k-halves are added through LDS at the end.
//
// Ring of P = 4 stages, one LDS array per stage so that the compiler's
// wait-count tracking tells the DMAs into one stage from reads of another:
//   X (16 KB): x in bf16 (rounded once into the workspace by x_to_bf16), row r
//              of the tile at byte 128 r, 16-byte chunk c at position c ^ (r & 7);
//   W (8 KB) : raw int8 rows, 64 bytes each, chunk c at position c ^ ((r >> 1) & 3);
//   D        : the stage's 256 scales (2 blocks x 128 rows) from the
//              block-major scale plane, four bytes per lane.
// Every lane of every wave issues the same four DMA instructions per stage
// (a DMA under a branch defeats the compiler's wait tracking), so the vmcnt
// waits are compile-time constants.  Stage s: issue the DMAs of stage s+3,
// read the fragments of stage s+1 and dequantise its B while the MFMAs of
// stage s run, wait until this wave's share of stage s+2 has landed, barrier.
// Each LDS read is one pointer step from its stage array (a 32-bit offset
// computed once), which keeps the access provably inside that array.
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

struct DmaArgs {
    const __bf16* xb;      // M x K bf16 (workspace)
    const int8_t* q;       // N x K int8 q plane (Q8_0 weights)
    const uint16_t* dT;    // (K/32) x N scales, block-major (Q8_0 weights)
    const __bf16* wb;      // N x K bf16 (the bf16 copy of dense f32 weights)
    float* out;            // M x N, or the slice partials part[slice][M][N]
    int64_t M, N, K, ntiles;
    int64_t kslice;        // K per slice (multiple of 64)
    int splits;
};

__global__ __launch_bounds__(256) void x_to_bf16(const float4* __restrict__ x, bf16x4* __restrict__ xb, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) xb[i] = to_bf16x4(x[i]);
}

// Stages of the LDS ring (as many as the 160 KB of LDS hold), each slot
// X | W | D: Q8_0 int8 rows and 512 B of scales (+ 256 B overflow); bf16 rows
constexpr int kDmaStagesQ8 = 4, kDmaStagesBf16 = 4;
template <bool BF16W>
constexpr int dma_slot() { return BF16W ? 16384 + 16384 : 16384 + 8192 + 768; }
template <bool BF16W>
constexpr int dma_stages() { return BF16W ? kDmaStagesBf16 : kDmaStagesQ8; }

// BF16W: the weights are bf16 rows laid out like x (no scales, nothing to
// dequantise: the B fragments are read as they stand), two DMAs a stage for
// them in place of the int8 rows and the scales, so every stage still has four.
template <bool BF16W>
__global__ __launch_bounds__(512) void gemm_dma(DmaArgs a)
{
    constexpr int P = dma_stages<BF16W>(), U = 2 * P, BM = 128, BN = 128;
    static_assert(P >= 4 && P <= 6, "ring of 4..6 stage arrays");
    constexpr int SLOT = dma_slot<BF16W>();
    constexpr int SLOT4 = P > 4 ? SLOT : 16, SLOT5 = P > 5 ? SLOT : 16;
    __shared__ __attribute__((aligned(1024))) char S0[SLOT], S1[SLOT], S2[SLOT], S3[SLOT], S4[SLOT4], S5[SLOT5];
#define QDEC_SLOT(u) ((u) == 0 ? S0 : (u) == 1 ? S1 : (u) == 2 ? S2 : (u) == 3 ? S3 : (u) == 4 ? S4 : S5)
    const int64_t id = blockIdx.x;
    const int64_t slice = id % a.splits, tile = id / a.splits;
    const int64_t n0 = (tile % a.ntiles) * BN, m0 = (tile / a.ntiles) * BM;
    const int64_t kbeg = slice * a.kslice;
    const int64_t klen = kbeg + a.kslice < a.K ? a.kslice : a.K - kbeg;
    const int ns = (int)(klen >> 6);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = wave >> 2, wn = wave & 3;

    // DMA sources at stage 0 of this slice (stage st adds 64 st elements)
    const __bf16* xsrc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (i * 8 + wave) * 8 + (lane >> 3);        // chunk slot (8i + wave)*64 + lane
        const int c = (lane & 7) ^ (r & 7);
        int64_t gr = m0 + r;
        gr = gr < a.M ? gr : a.M - 1;                          // rows past M repeat the last (never stored)
        xsrc[i] = a.xb + gr * a.K + kbeg + c * 8;
    }
    const int8_t* wsrc = nullptr;
    const __bf16* wbsrc[2] = {nullptr, nullptr};
    if constexpr (BF16W) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (i * 8 + wave) * 8 + (lane >> 3);    // as x, over the weight rows
            const int c = (lane & 7) ^ (r & 7);
            int64_t gn = n0 + r;
            gn = gn < a.N ? gn : a.N - 1;
            wbsrc[i] = a.wb + gn * a.K + kbeg + c * 8;
        }
    } else {
        const int r = wave * 16 + (lane >> 2);                 // chunk slot wave*64 + lane
        const int c = (lane & 3) ^ ((r >> 1) & 3);
        int64_t gn = n0 + r;
        gn = gn < a.N ? gn : a.N - 1;
        wsrc = a.q + gn * a.K + kbeg + c * 16;
    }
    // scales: word w*16 + L holds block (L%16)/8, rows 16(w + L/16) + 2(L%8)
    // + {0,1}: lanes L >= 16 write the words of the next waves, with the same
    // values those waves write (words past 127 land in the overflow)
    const uint16_t* dsrc = nullptr;
    if constexpr (!BF16W) {
        const int vw = wave + (lane >> 4), vl = lane & 15;
        int64_t gn = n0 + vw * 16 + 2 * (vl & 7);
        gn = gn < a.N - 1 ? gn : a.N - 2;                      // N even: pairs never straddle the edge
        dsrc = a.dT + (kbeg / 32 + (vl >> 3)) * a.N + gn;
    }
    auto issue = [&](int st, int u) {
        const int sc = st < ns ? st : ns - 1;                  // past the end: reload the last stage
        char* sb = QDEC_SLOT(u);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(xsrc[i] + (int64_t)sc * 64, (lds_void*)(sb + (i * 8 + wave) * 1024), 16, 0, 0);
        if constexpr (BF16W) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_amdgcn_global_load_lds(wbsrc[i] + (int64_t)sc * 64,
                                                 (lds_void*)(sb + 16384 + (i * 8 + wave) * 1024), 16, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds(wsrc + (int64_t)sc * 64, (lds_void*)(sb + 16384 + wave * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(dsrc + (int64_t)sc * 2 * a.N, (lds_void*)(sb + 24576 + wave * 64), 4, 0, 0);
        }
    };
    // fragment offsets inside a stage array (bytes)
    uint32_t xoff[8], woff[2], doff[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = i * 16 + (lane & 15);
        xoff[i] = r * 128 + (((uint32_t)wk * 4 + (lane >> 4)) ^ (r & 7)) * 16;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t r = wn * 32 + j * 16 + (lane & 15);
        if constexpr (BF16W) {
            woff[j] = 16384 + r * 128 + (((uint32_t)wk * 4 + (lane >> 4)) ^ (r & 7)) * 16;
            doff[j] = 0;
        } else {
            const uint32_t kb = wk * 32 + (lane >> 4) * 8;     // byte of the 64-byte row
            woff[j] = 16384 + r * 64 + ((kb >> 4) ^ ((r >> 1) & 3)) * 16 + (kb & 8);
            doff[j] = 24576 + 2 * ((r >> 4) * 32 + wk * 16 + (r & 15));
        }
    }
    bf16x8 fa[2][8], fb[2][2];
    u32x2 fq[2][2];
    uint16_t fd[2][2];
    auto frags = [&](int u, int f) {
        const char* sb = QDEC_SLOT(u);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (BF16W) {
                fb[f][j] = *reinterpret_cast<const bf16x8*>(sb + woff[j]);
            } else {
                fq[f][j] = *reinterpret_cast<const u32x2*>(sb + woff[j]);
                fd[f][j] = *reinterpret_cast<const uint16_t*>(sb + doff[j]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[f][i] = *reinterpret_cast<const bf16x8*>(sb + xoff[i]);
    };
    // B fragment j of set f: 8 weights d * q of one row, exact in f32, rounded to bf16
    auto deq = [&](int f, int j) -> bf16x8 {
        const float d = fp16_bits_to_f32(fd[f][j]);
        const uint32_t w[2] = {fq[f][j][0], fq[f][j][1]};
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)(d * (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xff));
        return v;
    };
    f32x4 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // prologue: stages 0..P-2 in flight; 0 and 1 landed everywhere; stage 0's
    // fragments read and dequantised
#pragma unroll
    for (int st = 0; st < P - 1; ++st) issue(st, st);
    wait_vm<4 * (P - 3)>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(0, 0);
    if constexpr (!BF16W) {
        fb[0][0] = deq(0, 0);
        fb[0][1] = deq(0, 1);
    }
    auto body = [&](const int s, const int u) {
        issue(s + P - 1, (u + P - 1) % P);
        const int f = u & 1;
        frags((u + 1) % P, f ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[f][i], fb[f][j], acc[i][j], 0, 0, 0);
        if constexpr (!BF16W) {
            fb[f ^ 1][0] = deq(f ^ 1, 0);
            fb[f ^ 1][1] = deq(f ^ 1, 1);
        }
        // this wave's share of stage s+2 has landed; the barrier makes every
        // wave's share visible and frees stage s-1's array for reuse
        wait_vm<4 * (P - 3)>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    int s0 = 0;
    for (; s0 + U <= ns; s0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) body(s0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (s0 + u < ns) body(s0 + u, u);
    wait_vm<0>();   // no DMA may still be writing LDS when it is reused or the workgroup ends
    __syncthreads();

    // the two k-halves: waves wk = 1 write their 128 x 32 partial tile (16 KB
    // each, one stage array per wave) and waves wk = 0 add it
    auto red = [&](int idx) -> f32x4* { return reinterpret_cast<f32x4*>(QDEC_SLOT(wn)) + idx; };
    if (wk == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) *red((i * 2 + j) * 64 + lane) = acc[i][j];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] += *red((i * 2 + j) * 64 + lane);
    // D layout of the 16x16 MFMA: lane holds column lane % 16, rows 4 (lane / 16) + e
    float* dst = a.out + (a.splits > 1 ? slice * a.M * a.N : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 32 + j * 16 + (lane & 15);
            if (n >= a.N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + i * 16 + (lane >> 4) * 4 + e;
                if (m < a.M) dst[m * a.N + n] = acc[i][j][e];
            }
        }
    }
#undef QDEC_SLOT
}

// out = sum over the K slices of their partial products, slice 0 first (a
// fixed order: the split result is reproducible, unlike atomic adds).
__global__ __launch_bounds__(256) void sum_slices(const float* __restrict__ part, int splits, int64_t mn,
                                                  float* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = mn / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 t = reinterpret_cast<const float4*>(part)[i];
        for (int sl = 1; sl < splits; ++sl) {
            const float4 u = reinterpret_cast<const float4*>(part + sl * mn)[i];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        reinterpret_cast<float4*>(out)[i] = t;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
        float t = part[i];
        for (int sl = 1; sl < splits; ++sl) t += part[sl * mn + i];
        out[i] = t;
    }
}

// The DMA-fed kernel holds ~135 KB of LDS: one workgroup per CU.  K is split
// into up to 8 slices (whole 64-k stages, at least 8 per slice) until the grid
// reaches about 192 workgroups; more slices cost more in partial products than
// the extra CUs give (measured: 128x8192x3072 split 3: 23.7 us, split 4: 24.7;
// 512x3072x8192 split 2: 47.3 us, split 4: 54.8).
int dma_splits(int64_t M, int64_t N, int64_t K)
{
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t stages = K / 64;
    int s = 1;
    while (s < 8 && tiles * (s + 1) <= 192 && stages / (s + 1) >= 8) ++s;
    return s;
}

bool dma_ok(int64_t N, int64_t K) { return K % 64 == 0 && N % 2 == 0 && N >= 2; }

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
    if (a.splits > 1 && !a.part) {
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
    if (a.splits > 1 && a.part) {
        const int64_t mn = a.M * a.N;
        int64_t sb = (mn / 4 + 255) / 256;
        if (sb > 2048) sb = 2048;
        if (sb < 1) sb = 1;
        hipLaunchKernelGGL(sum_slices, dim3((unsigned)sb), dim3(256), 0, s, a.part, a.splits, mn, a.out);
        count_launch();
    }
    return hipGetLastError();
}

// Register-staged path: the slices' partial products (none without a K split).
int64_t reg_part_bytes(int64_t M, int64_t N, int64_t K)
{
    const GemmArgs a = plan(M, N, K);
    return a.splits > 1 ? (int64_t)a.splits * M * N * 4 : 0;
}

}  // namespace

// x rounded to bf16, then (with a K split) the slices' partial products.
static int64_t dma_x_bytes(int64_t n_in, int64_t batch) { return align_up(batch * n_in * 2, kAlign); }

// K per slice of the DMA-fed kernel: whole 64-k stages, the last slice shorter.
static int64_t dma_kslice(int64_t K, int splits) { return (K / 64 + splits - 1) / splits * 64; }

int64_t q8_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch)
{
    if (!dma_ok(n_out, n_in)) return reg_part_bytes(batch, n_out, n_in);
    const int s = dma_splits(batch, n_out, n_in);
    return dma_x_bytes(n_in, batch) + (s > 1 ? (int64_t)s * batch * n_out * 4 : 0);
}

hipError_t launch_to_bf16(const float* src, int64_t count, void* dst, hipStream_t s)
{
    const int64_t n4 = count / 4;   // count % 4 == 0 (n_in % 32 == 0)
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(x_to_bf16, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(src),
                       static_cast<bf16x4*>(dst), n4);
    count_launch();
    return hipGetLastError();
}

int64_t f32_gemm_workspace_bytes(int64_t n_in, int64_t n_out, int64_t batch, bool bf16_copy)
{
    if (!bf16_copy || n_in % 64) return reg_part_bytes(batch, n_out, n_in);
    const int s = dma_splits(batch, n_out, n_in);
    return dma_x_bytes(n_in, batch) + (s > 1 ? (int64_t)s * batch * n_out * 4 : 0);
}

// Host-side extent checks of the plans below: the last element each kernel
// instance reads or writes, worked out again from the plan and the kernels'
// index formulas, against the extents of x, W, the scale plane, the
// workspace and out.  "" when every access stays inside.
static std::string gemm_over(const char* what, int64_t end, int64_t size)
{
    char why[256];
    std::snprintf(why, sizeof why, "batched GEMM plan: %s ends at %lld, extent %lld", what, (long long)end,
                  (long long)size);
    return std::string(why);
}

static std::string dma_plan_check(int64_t M, int64_t N, int64_t K, bool q8, int64_t ws_bytes)
{
    if (K % 64 || (q8 && (N % 2 || N < 2))) return gemm_over("K % 64 / even N", K, 0);
    const int splits = dma_splits(M, N, K);
    const int64_t kslice = dma_kslice(K, splits), nsl = (K + kslice - 1) / kslice;
    if (kslice <= 0 || kslice % 64) return gemm_over("K slice", kslice, K);
    if (nsl > splits) return gemm_over("slices", nsl, splits);
    // the last slice starts inside K and its stages end exactly at K
    const int64_t kbeg = (nsl - 1) * kslice, klen = K - kbeg;
    if (klen <= 0 || klen > kslice || klen % 64) return gemm_over("last slice", kbeg + klen, K);
    const int64_t ns = klen / 64;
    // x (bf16, workspace) and W rows: row clamped to M-1 / N-1, the last
    // stage's chunk 7 (bf16) or 3 (int8) of the last slice
    const int64_t x_end = (M - 1) * K + kbeg + (ns - 1) * 64 + 7 * 8 + 8;
    if (x_end > M * K) return gemm_over("x (bf16)", x_end, M * K);
    if (2 * M * K > dma_x_bytes(K, M)) return gemm_over("x in the workspace (bytes)", 2 * M * K, dma_x_bytes(K, M));
    const int64_t w_end = (N - 1) * K + kbeg + (ns - 1) * 64 + (q8 ? 3 * 16 + 16 : 7 * 8 + 8);
    if (w_end > N * K) return gemm_over("W rows", w_end, N * K);
    if (q8) {
        // block-major scales: block kbeg/32 + 1 + 2 (ns - 1) of row pair N-2, N-1
        const int64_t d_end = (kbeg / 32 + 1 + 2 * (ns - 1)) * N + (N - 2) + 2;
        if (d_end > (K / 32) * N) return gemm_over("scale plane", d_end, (K / 32) * N);
    }
    const int64_t grid = ((M + 127) / 128) * ((N + 127) / 128) * nsl;
    if (grid > INT32_MAX) return gemm_over("grid", grid, INT32_MAX);
    if (nsl > 1) {
        const int64_t need = dma_x_bytes(K, M) + nsl * M * N * 4;
        if (need > ws_bytes) return gemm_over("slice partials (bytes)", need, ws_bytes);
    } else if (dma_x_bytes(K, M) > ws_bytes) {
        return gemm_over("workspace (bytes)", dma_x_bytes(K, M), ws_bytes);
    }
    return std::string();
}

static std::string reg_plan_check(int64_t M, int64_t N, int64_t K, int64_t ws_bytes)
{
    const GemmArgs a = plan(M, N, K);
    if (a.kslice <= 0 || a.kslice % BK) return gemm_over("K slice", a.kslice, K);
    if ((int64_t)(a.splits - 1) * a.kslice >= K || (int64_t)a.splits * a.kslice < K)
        return gemm_over("slices x K slice", (int64_t)a.splits * a.kslice, K);
    if (a.mtiles * a.ntiles * a.splits > INT32_MAX) return gemm_over("grid", a.mtiles * a.ntiles * a.splits, INT32_MAX);
    // partials go to the workspace when there is one (else atomics into out)
    if (a.splits > 1 && ws_bytes > 0 && (int64_t)a.splits * M * N * 4 > ws_bytes)
        return gemm_over("slice partials (bytes)", (int64_t)a.splits * M * N * 4, ws_bytes);
    return std::string();
}

std::string q8_gemm_plan_check(int64_t n_in, int64_t n_out, int64_t batch, int64_t ws_bytes)
{
    if (ws_bytes > 0 && dma_ok(n_out, n_in)) return dma_plan_check(batch, n_out, n_in, true, ws_bytes);
    return reg_plan_check(batch, n_out, n_in, ws_bytes);
}

std::string f32_gemm_plan_check(int64_t n_in, int64_t n_out, int64_t batch, bool bf16_copy, int64_t ws_bytes)
{
    if (bf16_copy && ws_bytes > 0 && n_in % 64 == 0) return dma_plan_check(batch, n_out, n_in, false, ws_bytes);
    return reg_plan_check(batch, n_out, n_in, ws_bytes);
}

hipError_t launch_q8_0_gemm(Q8View w, int64_t n_in, int64_t n_out, int64_t batch, const float* x,
                            float* out, void* workspace, hipStream_t s)
{
    if (!q8_gemm_plan_check(n_in, n_out, batch, workspace ? q8_gemm_workspace_bytes(n_in, n_out, batch) : 0).empty())
        return hipErrorInvalidConfiguration;
    if (workspace && dma_ok(n_out, n_in)) {
        const int64_t n4 = batch * n_in / 4;   // n_in % 64 == 0
        int64_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(x_to_bf16, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(x),
                           static_cast<bf16x4*>(workspace), n4);
        count_launch();
        DmaArgs p{};
        p.xb = static_cast<const __bf16*>(workspace);
        p.q = w.q;
        p.dT = w.dT;
        p.M = batch;
        p.N = n_out;
        p.K = n_in;
        p.ntiles = (n_out + 127) / 128;
        const int splits = dma_splits(batch, n_out, n_in);
        p.kslice = dma_kslice(n_in, splits);
        p.splits = (int)((n_in + p.kslice - 1) / p.kslice);
        float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + dma_x_bytes(n_in, batch));
        p.out = p.splits > 1 ? part : out;
        const int64_t grid = ((batch + 127) / 128) * p.ntiles * p.splits;
        hipLaunchKernelGGL(gemm_dma<false>, dim3((unsigned)grid), dim3(512), 0, s, p);
        count_launch();
        if (p.splits > 1) {
            const int64_t mn = batch * n_out;
            int64_t sb = (mn / 4 + 255) / 256;
            if (sb > 2048) sb = 2048;
            if (sb < 1) sb = 1;
            hipLaunchKernelGGL(sum_slices, dim3((unsigned)sb), dim3(256), 0, s, part, p.splits, mn, out);
            count_launch();
        }
        return hipGetLastError();
    }
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.q = w.q;
    a.d = w.d;
    a.out = out;
    // a workspace given for a shape off the DMA-fed path holds the slices'
    // partial products (q8_gemm_workspace_bytes sized it)
    a.part = workspace && a.splits > 1 && !dma_ok(n_out, n_in) ? static_cast<float*>(workspace) : nullptr;
    return launch(a, true, s);
}

hipError_t launch_f32_gemm(const float* wf, const void* wbf16, int64_t n_in, int64_t n_out, int64_t batch,
                           const float* x, float* out, void* workspace, hipStream_t s)
{
    const bool copy = wbf16 != nullptr;
    if (!f32_gemm_plan_check(n_in, n_out, batch, copy,
                             workspace ? f32_gemm_workspace_bytes(n_in, n_out, batch, copy) : 0).empty())
        return hipErrorInvalidConfiguration;
    if (wbf16 && workspace && n_in % 64 == 0) {
        // the weight's bf16 copy (qdec_prepare): the DMA-fed kernel reads it
        // as it reads x
        const int64_t n4 = batch * n_in / 4;
        int64_t blocks = (n4 + 255) / 256;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(x_to_bf16, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(x),
                           static_cast<bf16x4*>(workspace), n4);
        count_launch();
        DmaArgs p{};
        p.xb = static_cast<const __bf16*>(workspace);
        p.wb = static_cast<const __bf16*>(wbf16);
        p.M = batch;
        p.N = n_out;
        p.K = n_in;
        p.ntiles = (n_out + 127) / 128;
        const int splits = dma_splits(batch, n_out, n_in);
        p.kslice = dma_kslice(n_in, splits);
        p.splits = (int)((n_in + p.kslice - 1) / p.kslice);
        float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + dma_x_bytes(n_in, batch));
        p.out = p.splits > 1 ? part : out;
        const int64_t grid = ((batch + 127) / 128) * p.ntiles * p.splits;
        hipLaunchKernelGGL(gemm_dma<true>, dim3((unsigned)grid), dim3(512), 0, s, p);
        count_launch();
        if (p.splits > 1) {
            const int64_t mn = batch * n_out;
            int64_t sb = (mn / 4 + 255) / 256;
            if (sb > 2048) sb = 2048;
            if (sb < 1) sb = 1;
            hipLaunchKernelGGL(sum_slices, dim3((unsigned)sb), dim3(256), 0, s, part, p.splits, mn, out);
            count_launch();
        }
        return hipGetLastError();
    }
    GemmArgs a = plan(batch, n_out, n_in);
    a.x = x;
    a.wf = wf;
    a.out = out;
    a.part = workspace && a.splits > 1 ? static_cast<float*>(workspace) : nullptr;
    return launch(a, false, s);
}

}  // namespace qdec
